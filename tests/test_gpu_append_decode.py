"""gqa_append_decode (the append and the decode of one step in one launch)
against the two calls it stands for, gqa_append_kv then gqa_decode, on the
same inputs: the output and the whole cache bitwise equal, and the output
within the usual tolerances of the oracle.  Cases cover the matrix-core
decode (one launch: head sizes 64/128/256, one to 70 new tokens, so that
new rows fill several units and two units of one wave, windows, sinks,
softcap, a rolling cache whose new rows wrap, lengths that skip a batch;
the call is checked to have run on the matrix cores) and the paths that run the append kernel first (fp32, more row tiles
than one launch takes)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan, oracle_decode
from windowed_gqa_kv_amd import binding
from windowed_gqa_kv_amd.inputs import WORKLOADS, Workload, generate, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    WORKLOADS[2],
    WORKLOADS[4].with_(Lk=20000, seqlens=("const", 16387)),
    Workload("ad", "decode", "f16", B=3, Hq=8, Hkv=2, D=64, Lq=3, Lk=700, window=200, head_sink=True,
             seqlens=("list", [2, 350, 699]), seed=5501),
    Workload("ad", "decode", "bf16", B=4, Hq=16, Hkv=4, D=128, Lq=16, Lk=900, window=-1, softcap=20.0,
             smooth_softmax=True, seqlens=("list", [15, 899, 500, 900]), seed=5502),  # batch 3 skipped
    Workload("ad", "decode", "f32", B=2, Hq=4, Hkv=2, D=64, Lq=2, Lk=300, window=50,
             seqlens=("list", [1, 200]), seed=5503),
    # new rows spanning several 16-key units (and, at 70, two units of one wave), five row tiles;
    # at 70 the first batch's cache holds only the new rows
    Workload("ad", "decode", "bf16", B=2, Hq=8, Hkv=4, D=128, Lq=40, Lk=1200, window=-1,
             seqlens=("list", [100, 1199]), seed=5505),
    Workload("ad", "decode", "f16", B=2, Hq=4, Hkv=4, D=256, Lq=70, Lk=3000, window=500, head_sink=True,
             seqlens=("list", [69, 2999]), seed=5506),
    Workload("ad", "decode", "bf16", B=33, Hq=64, Hkv=16, D=64, Lq=16, Lk=80, window=24, head_sink=True,
             seqlens=("uniform", 15, 80), seed=5504),  # 2112 row tiles: append kernel, then the decode
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.dtype}_D{w.D}_B{w.B}_c{w.Lq}_W{w.window}")
def test_append_decode_equals_append_then_decode(gpu, w):
    d = generate(w)
    plan = make_plan(w)
    q, kn, vn, seq = d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), d["seqlens_k"].cuda()
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    kc1, vc1 = d["k_cache"].cuda(), d["v_cache"].cuda()
    kc2, vc2 = kc1.clone(), vc1.clone()
    ws = plan.new_workspace()
    plan.append_kv(kn, vn, kc1, vc1, seq)
    out1 = plan.decode(q, kc1, vc1, seq, head_sink=sink, workspace=ws)
    out2 = plan.append_decode(q, kn, vn, kc2, vc2, seq, head_sink=sink, workspace=ws)
    path = binding.gqa_last_path()
    torch.cuda.synchronize()
    row_tiles = w.B * w.Hkv * -(-(w.Lq * (w.Hq // w.Hkv)) // 16)
    if w.dtype != "f32" and row_tiles <= 2048:
        assert path == binding.GQA_PATH_MATRIX_DECODE, binding.PATH_NAMES[path]
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2), "the caches differ"
    assert torch.equal(out1, out2), "the fused step's output differs from append + decode"
    s = d["seqlens_k"].numpy().astype(np.int64)
    ok = (s + 1 >= w.Lq) & (s + 1 <= w.Lk)
    if ok.all():
        compare(out2, oracle_decode(w, d), w.dtype, f"append_decode {w}")
    else:
        assert not out2[~torch.from_numpy(ok)].any(), "a batch with an out-of-range length must be 0"


def test_append_decode_rolling_wrap(gpu):
    """A rolling cache of W + curr - 1 slots whose step's new rows wrap past
    the ring's end: fused against the two calls, and against the oracle's
    ring."""
    W, curr = 100, 4
    C = W + curr - 1
    w = Workload("adr", "decode", "bf16", B=2, Hq=8, Hkv=2, D=128, Lq=curr, Lk=C, window=W,
                 seqlens=("list", [5 * C + 1, 3 * C + C - 2]), seed=5505)
    d = generate(w)
    plan = make_plan(w, rolling_cache=True)
    q, kn, vn, seq = d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), d["seqlens_k"].cuda()
    kc1, vc1 = d["k_cache"].cuda(), d["v_cache"].cuda()
    kc2, vc2 = kc1.clone(), vc1.clone()
    plan.append_kv(kn, vn, kc1, vc1, seq)
    out1 = plan.decode(q, kc1, vc1, seq)
    out2 = plan.append_decode(q, kn, vn, kc2, vc2, seq)
    torch.cuda.synchronize()
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    assert torch.equal(out1, out2)
    s = d["seqlens_k"].numpy().astype(np.int64)
    kr, vr = oracle.rolling.append(to_f64(d["k_cache"]), to_f64(d["v_cache"]), to_f64(d["k_new"]),
                                   to_f64(d["v_new"]), s)
    want = oracle.rolling.decode(to_f64(d["q"]), kr, vr, s, scale=w.sm_scale, window=W)
    compare(out2, want, "bf16", "rolling append_decode")
