"""The online softmax's lazy rescale on the GPU.

Both matrix-core kernels keep a running maximum per query row and move it only
when a new score tile (prefill: 64 keys; decode: a 16-key unit, each wave
taking every fourth unit of its slice) raises it by more than 2^8 in
exponential units, i.e. by more than 8 ln 2 = 5.545 nats of scaled (or capped)
logit.  The move rescales the row's denominator and its unnormalized output by
exp(old max - new max).  Seeded N(0,1) inputs keep logits within a few units,
so here the inputs are shaped (windowed_gqa_kv_amd.inputs.shape_logits) so that
every query's logit against key position j is about a prescribed level:
staircases and bursts that rise by 6.5-7.5 nats along the row.

Before the GPU runs, each test shows on the CPU, from the exact (rounded)
inputs, that the rescale must fire with a non-zero running sum and output:

* prefill: a row's first tile holds only keys among its first 64 allowed ones,
  so if the row's largest logit exceeds the largest of those by more than the
  threshold, some later tile moves the running max of a non-empty state;
* decode: a wave's consecutive units are 64 keys apart; if a unit's largest
  logit exceeds that of every earlier unit of the same residue by more than
  the threshold, the unit moves the running max whenever its wave streamed one
  of them before in the same slice.  Every slice holds at least 8 units (at
  least 16 units per workgroup on average, at least 8 in every tile), so the
  first slice of every tile holds units 0..7 and units 4..7 must fire.

Outputs are then compared with the float64 oracle at the usual tolerances.
Values change sign between levels, so an output that weighs the levels
wrongly is off by far more than the tolerance.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan, oracle_decode, oracle_prefill
from windowed_gqa_kv_amd.inputs import (Workload, bursts, generate, shape_logits, staircase,
                                        to_f64)

pytestmark = pytest.mark.gpu

THRESHOLD = 8.0 * math.log(2.0)  # nats of scaled (or capped) logit
MARGIN = 0.3
DECODE_GRID_MAX = 512             # workgroups of the decode grid (two per CU, 256 CUs)


def _capped(x, softcap):
    return softcap * np.tanh(x / softcap) if softcap > 0 else x


def _prefill_fire_fraction(w, d, mask=None):
    """Fraction of rows (with more than 64 allowed keys) whose largest logit
    exceeds the largest over their first 64 allowed keys by the threshold."""
    q, k = to_f64(d["q"]), to_f64(d["k"])
    G = w.Hq // w.Hkv
    nonpad = None if d.get("nonpad") is None else d["nonpad"].numpy()
    j = np.arange(w.Lk)
    fired = total = 0
    for b in range(w.B):
        valid = w.Lk if nonpad is None else int(nonpad[b])
        for h in range(w.Hq):
            x = w.sm_scale * (q[b, h] @ k[b, h // G].T)
            p = (w.Lk - w.Lq) + np.arange(w.Lq)
            M = oracle.allowed(p[:, None], j[None, :], valid, w.causal, w.window)
            if mask is not None:
                mb = np.broadcast_to(mask, (w.B, w.Hq, w.Lq, w.Lk))[b, h]
                if mb.dtype == np.bool_:
                    M = M & mb
                else:
                    M = M & (mb > -np.inf)
                    x = x + np.where(M, mb, 0.0)
            x = np.where(M, _capped(x, w.softcap), -np.inf)
            cnt = np.cumsum(M, axis=1)
            first = np.where(M & (cnt <= 64), x, -np.inf).max(axis=1)
            rows = cnt[:, -1] > 64
            with np.errstate(invalid="ignore"):
                rise = x.max(axis=1) - first
            fired += int(((rise > THRESHOLD + MARGIN) & rows).sum())
            total += int(rows.sum())
    return fired / max(total, 1)


def _decode_tiles(w, seqlens, masked=False):
    """(b, g, first row, rows, lo, hi) of every 16-row tile of the decode split.
    Row r of KV head g is query head g*G + r % G at new token r // G; a
    tile's keys are the union of its rows' allowed intervals (starting at a
    multiple of 16 keys with a caller mask)."""
    G = w.Hq // w.Hkv
    rows = G * w.Lq
    out = []
    for b in range(w.B):
        total = int(seqlens[b]) + 1
        q_off = total - w.Lq
        for g in range(w.Hkv):
            for r0 in range(0, rows, 16):
                nr = min(16, rows - r0)
                p0, p1 = q_off + r0 // G, q_off + (r0 + nr - 1) // G
                lo = 0 if w.window < 0 else max(0, p0 - w.window + 1)
                hi = p1 if w.causal else total - 1
                hi = min(hi, total - 1)
                if masked:
                    lo &= ~15
                out.append((b, g, r0, nr, lo, hi))
    return out


def _decode_fire_check(w, k_f64, q_f64, seqlens, mask=None):
    """Show that every tile's first slice must fire in units 4..7 (see the
    module docstring).  k_f64 is the dequantized cache after the append."""
    G = w.Hq // w.Hkv
    tiles = _decode_tiles(w, seqlens, masked=mask is not None)
    units = [(hi - lo) // 16 + 1 for (_, _, _, _, lo, hi) in tiles]
    assert sum(units) >= 16 * DECODE_GRID_MAX, "slices would hold fewer than 8 units"
    assert min(units) >= 8
    fired_rows = checked_rows = 0
    for (b, g, r0, nr, lo, hi), u in zip(tiles, units):
        total = int(seqlens[b]) + 1
        q_off = total - w.Lq
        for r in range(r0, r0 + nr):
            h, t = g * G + r % G, r // G
            p = q_off + t
            j = np.arange(lo, lo + 16 * 8)
            x = w.sm_scale * (k_f64[b, g, np.minimum(j, hi)] @ q_f64[b, h, t])
            ok = (j <= hi) & oracle.allowed(p, j, total, w.causal, w.window)
            if mask is not None:
                mb = np.broadcast_to(mask, (w.B, w.Hq, w.Lq, mask.shape[-1]))[b, h, t, np.minimum(j, mask.shape[-1] - 1)]
                if mb.dtype == np.bool_:
                    ok = ok & mb
                else:
                    ok = ok & (mb > -np.inf)
                    x = x + np.where(ok, mb, 0.0)
            x = np.where(ok, _capped(x, w.softcap), -np.inf).reshape(8, 16).max(axis=1)
            # unit 4 + i against unit i, for each of the four waves
            rises = x[4:8] - x[0:4]
            checked_rows += 1
            fired_rows += int(np.all(np.isfinite(x[0:4])) and np.all(rises > THRESHOLD + MARGIN))
    return fired_rows / checked_rows


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------
PREFILL = [
    # (id, dtype, D, Lq, Lk, window, softcap, sink, nonpad, profile, mask)
    ("stair_bf16_d128", "bf16", 128, 1024, 1024, -1, 0.0, False, None, ("stair", 7.5, 64), None),
    ("stair_f16_d64_win", "f16", 64, 900, 900, 300, 0.0, True, (700,), ("stair", 7.5, 64), None),
    ("bursts_bf16_d128", "bf16", 128, 1024, 1024, -1, 0.0, False, None, ("bursts", 6.8, 256, 16), None),
    ("bursts_f16_d128_win", "f16", 128, 1000, 1000, 600, 0.0, True, None, ("bursts", 6.8, 256, 8), None),
    ("stair_bf16_d128_cap", "bf16", 128, 1024, 1024, -1, 60.0, False, None, ("stair", 7.0, 256), None),
    ("stair_bf16_d64_bool", "bf16", 64, 800, 800, -1, 0.0, False, None, ("stair", 7.5, 64), "bool"),
    ("bursts_bf16_d128_add", "bf16", 128, 768, 768, -1, 0.0, True, None, ("bursts", 6.8, 192, 16), "add"),
    ("stair_bf16_d128_bool_cap", "bf16", 128, 768, 768, 500, 80.0, False, None, ("stair", 7.0, 128), "bool"),
    ("stair_f16_d128_add_cap", "f16", 128, 768, 768, -1, 80.0, False, None, ("stair", 7.0, 128), "add"),
    ("stair_bf16_d256_win", "bf16", 256, 768, 768, 400, 0.0, True, None, ("stair", 7.5, 64), None),
    ("bursts_f16_d256_cap_bool", "f16", 256, 768, 768, -1, 80.0, False, None, ("bursts", 6.8, 192, 16), "bool"),
    ("stair_bf16_d32", "bf16", 32, 768, 768, -1, 0.0, False, None, ("stair", 7.5, 64), None),
    ("bursts_f16_d32_add", "f16", 32, 768, 768, 500, 0.0, True, None, ("bursts", 6.8, 256, 8), "add"),
]


def _levels(profile, n):
    if profile[0] == "stair":
        return staircase(n, profile[1], profile[2])
    return bursts(n, profile[1], profile[2], profile[3])


def _mask(kind, shape, seed):
    rng = np.random.default_rng(seed)
    if kind == "bool":
        return rng.random(shape) < 0.85
    m = (rng.standard_normal(shape) * 0.3).astype(np.float32)
    m[rng.random(shape) < 0.05] = -np.inf
    return m


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: c[0])
def test_prefill_lazy_rescale(gpu, case):
    cid, dt, D, Lq, Lk, W, cap, sink, nonpad, profile, mkind = case
    w = Workload("rescale", "prefill", dt, B=1, Hq=4, Hkv=2, D=D, Lq=Lq, Lk=Lk, window=W, softcap=cap,
                 head_sink=sink, nonpad=nonpad, seed=zlib.crc32(cid.encode()) % 10000)
    d = shape_logits(w, generate(w), _levels(profile, Lk), seed=len(cid) + D)
    mask = None if mkind is None else _mask(mkind, (1, 1, Lq, Lk), seed=D + Lk)
    frac = _prefill_fire_fraction(w, d, mask)
    print(f"{cid}: rows whose running max must move after their first tile: {frac:.2f}", flush=True)
    assert frac >= 0.5
    plan = make_plan(w)
    out = plan.prefill(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(),
                       nonpad_kv_seqlen=None if d["nonpad"] is None else d["nonpad"].cuda(),
                       head_sink=None if d["head_sink"] is None else d["head_sink"].cuda(),
                       mask=None if mask is None else torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    want = oracle.prefill(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), scale=w.sm_scale,
                          window=W, softcap=cap, head_sink=to_f64(d["head_sink"]),
                          nonpad_kv_seqlen=None if d["nonpad"] is None else d["nonpad"].numpy(),
                          mask=None if mask is None else (mask if mask.dtype == np.bool_
                                                          else mask.astype(np.float64)))
    mx, mn = compare(out, want, dt, cid)
    print(f"{cid}: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
DECODE = [
    # (id, dtype, D, B, Hq, Hkv, curr, cap, window, softcap, sink, seqlens, step, period, mask)
    ("stair_bf16_d128_c1", "bf16", 128, 8, 32, 8, 1, 4096, -1, 0.0, False, ("uniform", 3000, 4096), 7.5, 64, None),
    ("stair_f16_d64_c4", "f16", 64, 8, 16, 8, 4, 4096, -1, 0.0, True, ("uniform", 3500, 4096), 7.5, 64, None),
    ("stair_bf16_d256_c4_win", "bf16", 256, 4, 16, 8, 4, 8192, 4096, 0.0, True, ("const", 8191), 7.5, 64, None),
    ("stair_bf16_d256_c4_cap", "bf16", 256, 4, 16, 8, 4, 8192, 4096, 60.0, True, ("const", 8191), 7.0, 64, None),
    ("stair_bf16_d128_c1_bool", "bf16", 128, 8, 32, 8, 1, 4096, -1, 0.0, False, ("uniform", 3000, 4096), 7.5, 64, "bool"),
    ("stair_bf16_d128_c2_add", "bf16", 128, 8, 16, 8, 2, 4096, -1, 0.0, False, ("uniform", 3000, 4096), 7.5, 64, "add"),
]


def _decode_levels(n, step, period, softcap, lo):
    """A staircase that starts at position lo; with a softcap only the first
    four levels rise (the cap flattens higher ones)."""
    lv = staircase(n, step, period)
    lv = np.maximum(lv - step * (lo // period), 0.0)
    if softcap > 0:
        lv = np.minimum(lv, 4 * step)
    return lv


@pytest.mark.parametrize("case", DECODE, ids=lambda c: c[0])
def test_decode_lazy_rescale(gpu, case):
    cid, dt, D, B, Hq, Hkv, curr, cap_, W, softcap, sink, seqlens, step, period, mkind = case
    w = Workload("rescale", "decode", dt, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap_, window=W,
                 softcap=softcap, head_sink=sink, smooth_softmax=not sink, seqlens=seqlens,
                 seed=zlib.crc32(cid.encode()) % 10000)
    d0 = generate(w)
    s = d0["seqlens_k"].numpy().astype(np.int64)
    lo = 0 if W < 0 else max(0, int(s.min()) + 1 - curr - W + 1)
    d = shape_logits(w, d0, _decode_levels(cap_, step, period, softcap, lo), seed=D + curr)
    mask = None if mkind is None else _mask(mkind, (B, Hq, curr, cap_), seed=D + cap_)
    top = int(s.max()) + 1
    kc64, _ = oracle.append_kv(to_f64(d["k_cache"][:, :, :top]), to_f64(d["v_cache"][:, :, :top]),
                               to_f64(d["k_new"]), to_f64(d["v_new"]), s)
    frac = _decode_fire_check(w, kc64, to_f64(d["q"]), s, mask)
    print(f"{cid}: rows whose units 4..7 must move the running max: {frac:.2f}", flush=True)
    assert frac >= 0.5
    plan = make_plan(w)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq = d["seqlens_k"].cuda()
    plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq)
    out = plan.decode(d["q"].cuda(), kc, vc, seq,
                      head_sink=None if d["head_sink"] is None else d["head_sink"].cuda(),
                      mask=None if mask is None else torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    if mask is None:
        want = oracle_decode(w, d)
    else:
        kcf, vc64 = oracle.append_kv(to_f64(d["k_cache"]), to_f64(d["v_cache"]), to_f64(d["k_new"]),
                                     to_f64(d["v_new"]), s)
        want = oracle.decode(to_f64(d["q"]), kcf, vc64, s, scale=w.sm_scale, window=W, softcap=softcap,
                             smooth_softmax=not sink, head_sink=to_f64(d["head_sink"]),
                             mask=mask if mask.dtype == np.bool_ else mask.astype(np.float64))
    mx, mn = compare(out, want, dt, cid)
    print(f"{cid}: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)


def _codes(x, scale):
    return (x.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("D,curr,mkind", [(128, 1, None), (256, 4, None), (128, 1, "bool")])
def test_fp8_decode_lazy_rescale(gpu, D, curr, mkind):
    """The same on FP8 caches: sixteen levels (the codes keep three mantissa
    bits, so the keys stay small enough for the levels to survive)."""
    Hq, Hkv = (32, 8) if D == 128 else (16, 8)
    B = 8 if D == 128 else 4
    cap_ = 4096 if D == 128 else 8192
    seqlens = ("uniform", 3000, 4096) if D == 128 else ("const", 8191)
    W = -1 if D == 128 else 4096
    w = Workload("rescale8", "decode", "bf16", B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap_, window=W,
                 smooth_softmax=True, seqlens=seqlens, seed=77 + D)
    d0 = generate(w)
    s = d0["seqlens_k"].numpy().astype(np.int64)
    lo = 0 if W < 0 else max(0, int(s.min()) + 1 - curr - W + 1)
    lv = np.minimum(_decode_levels(cap_, 7.5, 64, 0.0, lo), 15 * 7.5)
    d = shape_logits(w, d0, lv, seed=D)
    ks, vs = 0.05, 0.01
    kc0, vc0 = _codes(d["k_cache"], ks), _codes(d["v_cache"], vs)
    kc_o, vc_o = oracle.fp8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s, ks, vs)
    mask = None if mkind is None else _mask(mkind, (B, Hq, curr, cap_), seed=D + 5)
    frac = _decode_fire_check(w, oracle.fp8.dequantize(kc_o, ks), to_f64(d["q"]), s, mask)
    print(f"fp8 D={D}: rows whose units 4..7 must move the running max: {frac:.2f}", flush=True)
    assert frac >= 0.5
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq = d["seqlens_k"].cuda()
    plan.append_kv_fp8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq, ks, vs)
    out = plan.decode_fp8(d["q"].cuda(), kc, vc, seq, ks, vs,
                          mask=None if mask is None else torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), kc_o)
    top = int(s.max()) + 1
    want = oracle.fp8.decode(to_f64(d["q"]), kc_o[:, :, :top], vc_o[:, :, :top], s, k_scale=ks, v_scale=vs,
                             scale=w.sm_scale, window=W, smooth_softmax=True,
                             mask=None if mask is None else mask[..., :top])
    mx, mn = compare(out, want, "bf16", f"fp8 D={D}")
    print(f"fp8 D={D} curr={curr} mask={mkind}: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)
