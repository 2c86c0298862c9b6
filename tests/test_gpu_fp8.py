"""FP8 (E4M3) KV caches on the GPU (gqa_append_kv_fp8, gqa_decode_fp8,
gqa_decode_fp8_masked) against the oracle's FP8 cache (oracle.fp8), on the
same seeded inputs.

Quantization is integer work: the cached codes must equal the oracle's bit
for bit, over every 16-bit value and several scales.  Decode compares with
the oracle's attention over the dequantized caches at the usual tolerance.
Past cache contents are drawn as float32 normals and encoded with torch's
float8_e4m3fn cast (a library routine; the values stay far inside the range).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan
from windowed_gqa_kv_amd.inputs import TORCH_DTYPES, Workload, generate, to_f64

pytestmark = pytest.mark.gpu


def _codes(x, scale):
    """Codes of x / scale (CPU float tensor) through torch's E4M3 cast."""
    return (x.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.37, 3.0, 1e-3])
def test_fp8_append_quantizes_every_value_bit_exactly(gpu, dtype, scale):
    D, Hkv = 128, 1
    if dtype == "f32":
        rng = np.random.default_rng(5)
        vals = np.concatenate([[np.inf, -np.inf, np.nan, 0.0, -0.0, 447.9, 448.5, 464.0, 500.0],
                               rng.standard_normal(30000) * 300, rng.standard_normal(30000) * 1e-3])
        x = torch.from_numpy(vals.astype(np.float32))
    else:
        bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
        x = bits.view(TORCH_DTYPES[dtype])
    n = x.numel() // D * D
    curr = n // D
    x = x[:n].reshape(1, Hkv, curr, D)
    w = Workload("fp8q", "decode", dtype, B=1, Hq=1, Hkv=Hkv, D=D, Lq=curr, Lk=curr,
                 seqlens=("list", [curr - 1]), seed=1)
    plan = make_plan(w)
    kc = torch.zeros(1, Hkv, curr, D, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    seq = torch.tensor([curr - 1], dtype=torch.int32, device="cuda")
    xd = x.cuda()
    plan.append_kv_fp8(xd, xd, kc, vc, seq, scale, 2.0 * scale)
    torch.cuda.synchronize()
    want_k = oracle.fp8.quantize(x.float().numpy(), scale)
    want_v = oracle.fp8.quantize(x.float().numpy(), 2.0 * scale)
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    bad = np.nonzero(got_k != want_k)
    assert bad[0].size == 0, f"{bad[0].size} K codes differ, e.g. x={x.numpy()[bad][:4]} " \
                             f"got={got_k[bad][:4]} want={want_k[bad][:4]}"
    assert np.array_equal(got_v, want_v)


CASES = [
    # (dtype, B, Hq, Hkv, D, curr, cap, window, softcap, sink, seqlens, k_scale, v_scale)
    ("bf16", 4, 32, 8, 128, 1, 2048, -1, 0.0, False, [2047, 5, 1000, 333], 0.05, 0.02),
    ("bf16", 3, 16, 8, 256, 4, 1200, 500, 50.0, True, [1199, 700, 3], 0.1, 0.1),
    ("f16", 2, 8, 2, 64, 3, 700, -1, 0.0, True, [699, 64], 0.02, 0.05),
    ("bf16", 2, 8, 1, 128, 2, 4096, 1000, 0.0, False, [4095, 2500], 1.0, 0.5),
    # 40 new rows: several units of new keys, five row tiles per head group
    ("bf16", 2, 8, 4, 128, 40, 1500, 300, 0.0, True, [1499, 39], 0.05, 0.05),
    ("f16", 2, 4, 2, 256, 40, 900, -1, 30.0, False, [899, 450], 0.1, 0.02),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_D{c[4]}_curr{c[5]}_W{c[7]}")
def test_fp8_append_and_decode_match_oracle(gpu, case):
    dtype, B, Hq, Hkv, D, curr, cap, W, cap_, sink, seq, ks, vs = case
    w = Workload("fp8dec", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap, window=W,
                 softcap=cap_, head_sink=sink, smooth_softmax=not sink, seqlens=("list", seq),
                 seed=600 + D + curr)
    d = generate(w)
    kc0, vc0 = _codes(d["k_cache"], ks), _codes(d["v_cache"], vs)
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_fp8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks, vs)
    out = plan.decode_fp8(d["q"].cuda(), kc, vc, seq_d, ks, vs,
                          head_sink=None if d["head_sink"] is None else d["head_sink"].cuda())
    torch.cuda.synchronize()
    s = np.asarray(seq, dtype=np.int64)
    kc_o, vc_o = oracle.fp8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s,
                                   ks, vs)
    assert np.array_equal(kc.cpu().numpy(), kc_o) and np.array_equal(vc.cpu().numpy(), vc_o)
    top = int(s.max()) + 1
    want = oracle.fp8.decode(to_f64(d["q"]), kc_o[:, :, :top], vc_o[:, :, :top], s, k_scale=ks, v_scale=vs,
                             scale=w.sm_scale, window=W, softcap=cap_, smooth_softmax=not sink,
                             head_sink=to_f64(d["head_sink"]))
    compare(out, want, dtype, f"fp8 decode {case}")


def test_fp8_decode_full_size_and_rolling(gpu):
    """The headline decode workload (8 x 32 heads, caches of 4096) on FP8
    caches against the oracle; then a rolling FP8 cache (window 1024 on a
    1024-slot ring, positions past it) against the oracle's ring."""
    from windowed_gqa_kv_amd.inputs import WORKLOADS
    w = WORKLOADS[2]
    d = generate(w)
    ks, vs = 0.03, 0.03
    kc0, vc0 = _codes(d["k_cache"], ks), _codes(d["v_cache"], vs)
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_fp8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks, vs)
    out = plan.decode_fp8(d["q"].cuda(), kc, vc, seq_d, ks, vs)
    torch.cuda.synchronize()
    s = d["seqlens_k"].numpy().astype(np.int64)
    top = int(s.max()) + 1
    kc_o, vc_o = oracle.fp8.append(kc0.numpy()[:, :, :top], vc0.numpy()[:, :, :top], to_f64(d["k_new"]),
                                   to_f64(d["v_new"]), s, ks, vs)
    want = oracle.fp8.decode(to_f64(d["q"]), kc_o, vc_o, s, k_scale=ks, v_scale=vs, scale=w.sm_scale,
                             smooth_softmax=True)
    compare(out, want, "bf16", "full-size fp8 decode")

    # rolling FP8 cache
    wr = Workload("fp8ring", "decode", "bf16", B=2, Hq=8, Hkv=2, D=128, Lq=1, Lk=1024, window=1024,
                  seqlens=("list", [5000, 1500]), seed=66)
    dr = generate(wr)
    plan = make_plan(wr, rolling_cache=True)
    kc0, vc0 = _codes(dr["k_cache"], ks), _codes(dr["v_cache"], vs)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = dr["seqlens_k"].cuda()
    plan.append_kv_fp8(dr["k_new"].cuda(), dr["v_new"].cuda(), kc, vc, seq_d, ks, vs)
    out = plan.decode_fp8(dr["q"].cuda(), kc, vc, seq_d, ks, vs)
    torch.cuda.synchronize()
    s = np.array([5000, 1500], dtype=np.int64)
    kq = oracle.fp8.quantize(to_f64(dr["k_new"]), ks).astype(np.float64)
    vq = oracle.fp8.quantize(to_f64(dr["v_new"]), vs).astype(np.float64)
    kr, vr = oracle.rolling.append(kc0.numpy().astype(np.float64), vc0.numpy().astype(np.float64), kq, vq, s)
    assert np.array_equal(kc.cpu().numpy(), kr.astype(np.uint8))
    want = oracle.rolling.decode(to_f64(dr["q"]), oracle.fp8.dequantize(kr.astype(np.uint8), ks),
                                 oracle.fp8.dequantize(vr.astype(np.uint8), vs), s, scale=wr.sm_scale,
                                 window=1024)
    compare(out, want, "bf16", "rolling fp8 decode")


@pytest.mark.parametrize("dtype,D,curr,cap,kind,softcap,ks", [
    ("bf16", 128, 1, 1024, "bool", 0.0, 0.05),
    ("bf16", 256, 4, 600, "add", 50.0, 0.1),
    ("f16", 64, 3, 800, "add", 0.0, 0.02),
    ("f16", 64, 2, 300, "bool", 5.0, 0.5),
])
def test_fp8_decode_with_mask_matches_oracle(gpu, dtype, D, curr, cap, kind, softcap, ks):
    """gqa_decode_fp8_masked against the oracle's attention over the
    dequantized caches with the same mask (an additive value joins the scaled
    logit of the dequantized K); a row whose mask removes every key is 0."""
    B, Hq, Hkv = 3, 8, 2
    seq = [cap - 1, 17, cap // 2]
    w = Workload("fp8mask", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap,
                 window=-1 if D != 256 else 200, softcap=softcap, smooth_softmax=True,
                 seqlens=("list", seq), seed=700 + D + curr)
    d = generate(w)
    vs = 0.03
    rng = np.random.default_rng(D + cap)
    shape = (B, Hq, curr, cap)
    if kind == "bool":
        mask = torch.from_numpy(rng.random(shape) < 0.6)
        mask[1, 3] = False
    else:
        m = (rng.standard_normal(shape) * 2.0).astype(np.float32)
        m[rng.random(shape) < 0.05] = -np.inf
        m[1, 3] = -np.inf
        mask = torch.from_numpy(m)
    kc0, vc0 = _codes(d["k_cache"], ks), _codes(d["v_cache"], vs)
    plan = make_plan(w)
    kc, vc = kc0.cuda(), vc0.cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv_fp8(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d, ks, vs)
    out = plan.decode_fp8(d["q"].cuda(), kc, vc, seq_d, ks, vs, mask=mask.cuda())
    torch.cuda.synchronize()
    s = np.asarray(seq, dtype=np.int64)
    kc_o, vc_o = oracle.fp8.append(kc0.numpy(), vc0.numpy(), to_f64(d["k_new"]), to_f64(d["v_new"]), s, ks, vs)
    want = oracle.fp8.decode(to_f64(d["q"]), kc_o, vc_o, s, k_scale=ks, v_scale=vs, scale=w.sm_scale,
                             window=w.window, softcap=softcap, smooth_softmax=True,
                             mask=mask.numpy() if kind == "bool" else mask.numpy().astype(np.float64))
    compare(out, want, dtype, f"fp8 masked decode {dtype} D={D} curr={curr} {kind}")
    assert not out[1, 3].any(), "a head whose mask removes every key must give 0"
