"""INT8 KV caches with per-KV-head scales on the GPU (gqa_append_kv_int8,
gqa_decode_int8, gqa_decode_int8_masked) against the oracle's INT8 cache
(oracle.int8), on the same seeded inputs.

Quantization is integer work: the cached codes must equal the oracle's bit
for bit, over every 16-bit value, with different scales per KV head.  Decode
compares with the oracle's attention over the dequantized caches at the
usual tolerance.  Past cache contents are codes drawn uniformly."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan
from windowed_gqa_kv_amd.inputs import TORCH_DTYPES, Workload, generate, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_int8_append_quantizes_every_value_bit_exactly(gpu, dtype):
    D, Hkv = 128, 2
    if dtype == "f32":
        rng = np.random.default_rng(6)
        vals = np.concatenate([[np.inf, -np.inf, np.nan, 0.0, -0.0, 0.5, 1.5, 2.5, -2.5, 127.4, 127.5, 200.0],
                               rng.standard_normal(30000) * 50, rng.standard_normal(30000) * 1e-2])
        x = torch.from_numpy(vals.astype(np.float32))
    else:
        x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(TORCH_DTYPES[dtype])
    n = x.numel() // (D * Hkv) * (D * Hkv)
    curr = n // (D * Hkv)
    x = x[:n].reshape(1, Hkv, curr, D)
    w = Workload("i8q", "decode", dtype, B=1, Hq=Hkv, Hkv=Hkv, D=D, Lq=curr, Lk=curr,
                 seqlens=("list", [curr - 1]), seed=1)
    plan = make_plan(w)
    ks = torch.tensor([0.37, 0.01], dtype=torch.float32)
    vs = torch.tensor([2.0, 0.05], dtype=torch.float32)
    kc = torch.zeros(1, Hkv, curr, D, dtype=torch.int8, device="cuda")
    vc = torch.zeros_like(kc)
    seq = torch.tensor([curr - 1], dtype=torch.int32, device="cuda")
    plan.append_kv_int8(x.cuda(), x.cuda(), kc, vc, seq, ks.cuda(), vs.cuda())
    torch.cuda.synchronize()
    want_k = oracle.int8.quantize(x.float().numpy(), ks.numpy())
    want_v = oracle.int8.quantize(x.float().numpy(), vs.numpy())
    bad = np.nonzero(kc.cpu().numpy() != want_k)
    assert bad[0].size == 0, f"{bad[0].size} K codes differ"
    assert np.array_equal(vc.cpu().numpy(), want_v)


CASES = [
    # (dtype, B, Hq, Hkv, D, curr, cap, window, softcap, sink, seqlens)
    ("bf16", 4, 32, 8, 128, 1, 2048, -1, 0.0, False, [2047, 5, 1000, 333]),
    ("bf16", 3, 16, 8, 256, 4, 1200, 500, 50.0, True, [1199, 700, 3]),
    ("f16", 2, 8, 2, 64, 3, 700, -1, 0.0, True, [699, 64]),
    ("bf16", 2, 8, 1, 128, 2, 4096, 1000, 0.0, False, [4095, 2500]),
    # 40 new rows: several units of new keys, five row tiles per head group
    ("bf16", 2, 8, 4, 128, 40, 1500, 300, 0.0, True, [1499, 39]),
    ("f16", 2, 4, 2, 256, 40, 900, -1, 30.0, False, [899, 450]),
]


def _scales(Hkv, seed, lo, hi):
    return torch.from_numpy(np.random.default_rng(seed).uniform(lo, hi, Hkv).astype(np.float32))


def _run(w, d, ks, vs):
    rng = np.random.default_rng(w.seed)
    kc0 = torch.from_numpy(rng.integers(-127, 128, (w.B, w.Hkv, w.Lk, w.D)).astype(np.int8))
    vc0 = torch.from_numpy(rng.integers(-127, 128, (w.B, w.Hkv, w.Lk, w.D)).astype(np.int8))
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_int8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda())
    out = plan.decode_int8(d["q"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda(),
                           head_sink=None if d["head_sink"] is None else d["head_sink"].cuda())
    torch.cuda.synchronize()
    s = d["seqlens_k"].numpy().astype(np.int64)
    kc_o, vc_o = oracle.int8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s,
                                    ks.numpy(), vs.numpy())
    assert np.array_equal(kc.cpu().numpy(), kc_o) and np.array_equal(vc.cpu().numpy(), vc_o)
    return out, kc_o, vc_o, s


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_D{c[4]}_curr{c[5]}_W{c[7]}")
def test_int8_append_and_decode_match_oracle(gpu, case):
    dtype, B, Hq, Hkv, D, curr, cap, W, cap_, sink, seq = case
    w = Workload("i8dec", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap, window=W,
                 softcap=cap_, head_sink=sink, smooth_softmax=not sink, seqlens=("list", seq),
                 seed=800 + D + curr)
    d = generate(w)
    # scales around max|x| / 127 of N(0,1) draws, different per KV head
    ks, vs = _scales(Hkv, D, 0.02, 0.06), _scales(Hkv, D + 1, 0.01, 0.05)
    out, kc_o, vc_o, s = _run(w, d, ks, vs)
    top = int(s.max()) + 1
    want = oracle.int8.decode(to_f64(d["q"]), kc_o[:, :, :top], vc_o[:, :, :top], s, k_scales=ks.numpy(),
                              v_scales=vs.numpy(), scale=w.sm_scale, window=W, softcap=cap_,
                              smooth_softmax=not sink, head_sink=to_f64(d["head_sink"]))
    compare(out, want, dtype, f"int8 decode {case}")


def test_int8_decode_full_size(gpu):
    """The headline decode workload (8 x 32 heads, caches of 4096) on INT8
    caches against the oracle."""
    from windowed_gqa_kv_amd.inputs import WORKLOADS
    w = WORKLOADS[2]
    d = generate(w)
    ks, vs = _scales(w.Hkv, 3, 0.025, 0.035), _scales(w.Hkv, 4, 0.025, 0.035)
    out, kc_o, vc_o, s = _run(w, d, ks, vs)
    top = int(s.max()) + 1
    want = oracle.int8.decode(to_f64(d["q"]), kc_o[:, :, :top], vc_o[:, :, :top], s, k_scales=ks.numpy(),
                              v_scales=vs.numpy(), scale=w.sm_scale, smooth_softmax=True)
    compare(out, want, "bf16", "full-size int8 decode")


def test_int8_decode_lazy_rescale(gpu):
    """Codes whose logits rise by 7.5 nats every 64 keys along the row (a
    staircase through the code range): the running max moves in every wave
    after its first unit, with a per-head K scale in the softmax scale."""
    w = Workload("i8resc", "decode", "bf16", B=8, Hq=32, Hkv=8, D=128, Lq=1, Lk=4096, window=-1,
                 smooth_softmax=True, seqlens=("uniform", 3000, 4096), seed=811)
    d = generate(w)
    rng = np.random.default_rng(12)
    ks = _scales(w.Hkv, 13, 0.8, 1.0)
    vs = _scales(w.Hkv, 14, 0.01, 0.02)
    u = rng.choice([-1.0, 1.0], size=w.D)
    q = torch.from_numpy((u[None, None, None, :] + 0.1 * rng.standard_normal((w.B, w.Hq, 1, w.D))).astype(np.float32))
    d["q"] = q.to(torch.bfloat16)
    # key at position j: code (j // 64) * c along u (logit ~ 7.5 per level), plus code noise
    s = d["seqlens_k"].numpy().astype(np.int64)
    lvl = np.arange(w.Lk) // 64
    ksn = ks.numpy()[None, :, None, None]
    # logit = scale * q.k = (1/sqrt(D)) * sum_d u_d * code_d * k_scale ~ sqrt(D) * code * k_scale
    code = np.clip(np.rint(lvl[None, None, :, None] * 7.5 / (np.sqrt(w.D) * ksn)), -120, 120)
    base = (code * u[None, None, None, :] + rng.integers(-1, 2, (w.B, w.Hkv, w.Lk, w.D))).clip(-127, 127)
    # the new token's row at its position, as values (quantized by the append)
    pos = s + 1 - 1
    kn = np.stack([base[b, :, pos[b]] for b in range(w.B)])[:, :, None, :] * ksn[0, :, 0, 0][None, :, None, None]
    d["k_new"] = torch.from_numpy(kn.astype(np.float32)).to(torch.bfloat16)
    kc0 = torch.from_numpy(base.astype(np.int8))
    vc0 = torch.from_numpy(rng.integers(-127, 128, (w.B, w.Hkv, w.Lk, w.D)).astype(np.int8))
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_int8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda())
    out = plan.decode_int8(d["q"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda())
    torch.cuda.synchronize()
    kc_o, vc_o = oracle.int8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s,
                                    ks.numpy(), vs.numpy())
    # the rise the test needs: unit 4 + i beats unit i by more than 8 ln 2 in every row
    kd = oracle.int8.dequantize(kc_o, ks.numpy())
    qd = to_f64(d["q"])
    x = np.einsum("bhd,bhjd->bhj", qd[:, :, 0], np.repeat(kd, w.Hq // w.Hkv, axis=1)[:, :, :128]) / np.sqrt(w.D)
    um = x.reshape(w.B, w.Hq, 8, 16).max(-1)
    assert (um[:, :, 4:8] - um[:, :, 0:4] > 8 * np.log(2) + 0.3).all()
    top = int(s.max()) + 1
    want = oracle.int8.decode(qd, kc_o[:, :, :top], vc_o[:, :, :top], s, k_scales=ks.numpy(),
                              v_scales=vs.numpy(), scale=w.sm_scale, smooth_softmax=True)
    compare(out, want, "bf16", "int8 rescale")


def test_int8_decode_rolling(gpu):
    """A rolling INT8 cache (window 600, three new tokens, a ring of
    W + curr - 1 = 602 slots, positions far past it, different scales per KV
    head): the ring after the step equals the oracle's bit for bit, and the
    decode matches the oracle's attention over the dequantized ring."""
    W, curr = 600, 3
    w = Workload("i8ring", "decode", "bf16", B=2, Hq=8, Hkv=2, D=256, Lq=curr, Lk=W + curr - 1, window=W,
                 softcap=30.0, head_sink=True, seqlens=("list", [5000, 1300]), seed=831)
    d = generate(w)
    rng = np.random.default_rng(832)
    kc0 = torch.from_numpy(rng.integers(-127, 128, (w.B, w.Hkv, w.Lk, w.D)).astype(np.int8))
    vc0 = torch.from_numpy(rng.integers(-127, 128, (w.B, w.Hkv, w.Lk, w.D)).astype(np.int8))
    ks, vs = _scales(w.Hkv, 833, 0.02, 0.06), _scales(w.Hkv, 834, 0.01, 0.05)
    plan = make_plan(w, rolling_cache=True)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_int8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda())
    out = plan.decode_int8(d["q"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda(), head_sink=d["head_sink"].cuda())
    torch.cuda.synchronize()
    s = d["seqlens_k"].numpy().astype(np.int64)
    kq = oracle.int8.quantize(to_f64(d["k_new"]), ks.numpy()).astype(np.float64)
    vq = oracle.int8.quantize(to_f64(d["v_new"]), vs.numpy()).astype(np.float64)
    kr, vr = oracle.rolling.append(kc0.numpy().astype(np.float64), vc0.numpy().astype(np.float64), kq, vq, s)
    assert np.array_equal(kc.cpu().numpy(), kr.astype(np.int8))
    assert np.array_equal(vc.cpu().numpy(), vr.astype(np.int8))
    want = oracle.rolling.decode(to_f64(d["q"]), oracle.int8.dequantize(kr.astype(np.int8), ks.numpy()),
                                 oracle.int8.dequantize(vr.astype(np.int8), vs.numpy()), s, scale=w.sm_scale,
                                 window=W, softcap=30.0, head_sink=to_f64(d["head_sink"]))
    compare(out, want, "bf16", "rolling int8 decode")


@pytest.mark.parametrize("dtype,D,curr,cap,kind,softcap", [
    ("bf16", 128, 1, 1024, "bool", 0.0),
    ("bf16", 256, 4, 600, "add", 50.0),
    ("f16", 64, 3, 800, "add", 0.0),
    ("f16", 64, 2, 300, "bool", 5.0),
])
def test_int8_decode_with_mask_matches_oracle(gpu, dtype, D, curr, cap, kind, softcap):
    """gqa_decode_int8_masked against the oracle's attention over the
    dequantized caches with the same mask: an additive value joins the scaled
    logit of the dequantized K whatever the head's k_scale (the scales differ
    by up to 5x between heads here), and a row whose mask removes every key
    is 0."""
    B, Hq, Hkv = 3, 8, 2
    seq = [cap - 1, 17, cap // 2]
    w = Workload("i8mask", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap,
                 window=-1 if D != 256 else 200, softcap=softcap, smooth_softmax=True,
                 seqlens=("list", seq), seed=850 + D + curr)
    d = generate(w)
    ks = torch.tensor([0.012, 0.06], dtype=torch.float32)
    vs = _scales(Hkv, D + 2, 0.01, 0.05)
    rng = np.random.default_rng(D + cap + 1)
    shape = (B, Hq, curr, cap)
    if kind == "bool":
        mask = torch.from_numpy(rng.random(shape) < 0.6)
        mask[1, 3] = False
    else:
        m = (rng.standard_normal(shape) * 2.0).astype(np.float32)
        m[rng.random(shape) < 0.05] = -np.inf
        m[1, 3] = -np.inf
        mask = torch.from_numpy(m)
    kc0 = torch.from_numpy(rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8))
    vc0 = torch.from_numpy(rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8))
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_int8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda())
    out = plan.decode_int8(d["q"].cuda(), kc, vc, seq_d, ks.cuda(), vs.cuda(), mask=mask.cuda())
    torch.cuda.synchronize()
    s = np.asarray(seq, dtype=np.int64)
    kc_o, vc_o = oracle.int8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s,
                                    ks.numpy(), vs.numpy())
    assert np.array_equal(kc.cpu().numpy(), kc_o) and np.array_equal(vc.cpu().numpy(), vc_o)
    want = oracle.int8.decode(to_f64(d["q"]), kc_o, vc_o, s, k_scales=ks.numpy(), v_scales=vs.numpy(),
                              scale=w.sm_scale, window=w.window, softcap=softcap, smooth_softmax=True,
                              mask=mask.numpy() if kind == "bool" else mask.numpy().astype(np.float64))
    compare(out, want, dtype, f"int8 masked decode {dtype} D={D} curr={curr} {kind}")
    assert not out[1, 3].any(), "a head whose mask removes every key must give 0"
