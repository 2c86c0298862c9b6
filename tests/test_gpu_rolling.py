"""Rolling (ring-buffer) KV cache on the GPU against the oracle's rolling cache
(oracle.rolling): gqa_append_kv writes a step into the slots of its
positions mod capacity, gqa_decode reads the key at position j from slot
j mod capacity, and the result is the windowed attention over the whole
history.  Positions run far past the capacity (the ring wrapped many times),
and the decode's split pieces cross the wrap.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan
from windowed_gqa_kv_amd.inputs import TORCH_DTYPES, Workload, generate, rotary_tables, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, B, Hq, Hkv, D, curr, W, capacity, seqlens_k, softcap, sink)
    ("bf16", 4, 32, 8, 128, 1, 2048, 2048, [9999, 12047, 10100, 14000], 0.0, False),
    ("bf16", 3, 16, 8, 256, 4, 1000, 1003, [1002, 5000, 3456], 50.0, True),
    ("bf16", 2, 8, 2, 128, 3, 300, 512, [1 << 20, (1 << 20) + 333], 0.0, True),
    ("f16", 2, 8, 8, 64, 2, 64, 65, [64, 1000], 0.0, False),
    ("f32", 2, 4, 2, 32, 2, 20, 21, [30, 5], 0.0, True),
    ("bf16", 2, 8, 2, 96, 1, 40, 40, [77, 39], 0.0, False),  # generic kernel (head size 96)
    # 40 new rows, at the smallest ring (W + curr - 1) and past it
    ("bf16", 2, 8, 2, 128, 40, 200, 239, [5000, 239], 0.0, True),
    ("bf16", 2, 8, 4, 256, 40, 100, 160, [3000, 1000], 30.0, False),
]


def _ids(c):
    return f"{c[0]}_D{c[4]}_curr{c[5]}_W{c[6]}_C{c[7]}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_rolling_append_and_decode_match_oracle(gpu, case):
    dtype, B, Hq, Hkv, D, curr, W, cap, seq, softcap, sink = case
    w = Workload("ring", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap, window=W,
                 softcap=softcap, head_sink=sink, smooth_softmax=not sink, seqlens=("list", seq),
                 seed=zlib.crc32(_ids(case).encode()) % 10000)
    d = generate(w)
    plan = make_plan(w, rolling_cache=True)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq_d = d["seqlens_k"].cuda()
    plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d)
    out = plan.decode(d["q"].cuda(), kc, vc, seq_d,
                      head_sink=None if d["head_sink"] is None else d["head_sink"].cuda())
    torch.cuda.synchronize()

    s = np.asarray(seq, dtype=np.int64)
    kr, vr = oracle.rolling.append(to_f64(d["k_cache"]), to_f64(d["v_cache"]), to_f64(d["k_new"]),
                                   to_f64(d["v_new"]), s)
    # the ring after the step, slot by slot (values are copies: bitwise)
    assert np.array_equal(to_f64(kc), kr) and np.array_equal(to_f64(vc), vr)
    want = oracle.rolling.decode(to_f64(d["q"]), kr, vr, s, scale=w.sm_scale, window=W,
                                 softcap=softcap, smooth_softmax=not sink,
                                 head_sink=to_f64(d["head_sink"]))
    compare(out, want, dtype, f"rolling decode {_ids(case)}")


def test_rolling_steps_over_many_wraps_match_full_history(gpu):
    """A ring filled by 40 consecutive single-token steps through the GPU
    path (the ring wraps four times), then compared with the windowed decode
    over the full history that the test keeps on the side."""
    B, Hq, Hkv, D, W, cap, steps = 2, 8, 2, 128, 10, 10, 40
    w = Workload("ringsteps", "decode", "bf16", B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=1, Lk=cap, window=W,
                 seqlens=("list", [0, 0]), seed=7)
    plan = make_plan(w, rolling_cache=True)
    rng = np.random.default_rng(11)
    hist_k = torch.from_numpy(rng.standard_normal((B, Hkv, steps, D), dtype=np.float32)).bfloat16()
    hist_v = torch.from_numpy(rng.standard_normal((B, Hkv, steps, D), dtype=np.float32)).bfloat16()
    kc = torch.zeros(B, Hkv, cap, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    hk, hv = hist_k.cuda(), hist_v.cuda()
    q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32)).bfloat16()
    ws = plan.new_workspace()
    for p in range(steps):
        seq = torch.full((B,), p, dtype=torch.int32, device="cuda")
        plan.append_kv(hk[:, :, p:p + 1].contiguous(), hv[:, :, p:p + 1].contiguous(), kc, vc, seq)
    out = plan.decode(q.cuda(), kc, vc, seq, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.decode(to_f64(q), to_f64(hist_k), to_f64(hist_v), np.full(B, steps - 1),
                         scale=w.sm_scale, window=W)
    compare(out, want, "bf16", "ring filled step by step")


def test_rolling_with_rotary(gpu):
    """Rotary and a rolling cache together: the new K rows are turned at their
    true positions (past the capacity) and written to their ring slots."""
    dtype, B, Hq, Hkv, D, curr, W, cap = "bf16", 2, 8, 2, 128, 2, 100, 101
    seq = [5000, 777]
    w = Workload("ringrot", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap, window=W,
                 smooth_softmax=True, seqlens=("list", seq), seed=23)
    d = generate(w)
    cos, sin = rotary_tables(6000, D)
    plan = make_plan(w, rolling_cache=True)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq_d = d["seqlens_k"].cuda()
    q_rot = plan.append_kv_rotary(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d,
                                  cos.cuda(), sin.cuda())
    out = plan.decode(q_rot, kc, vc, seq_d)
    torch.cuda.synchronize()

    s = np.asarray(seq, dtype=np.int64)
    pos = oracle.rotary.decode_positions(s, curr)[:, None, :]
    c64, s64 = to_f64(cos), to_f64(sin)
    rnd = lambda x: torch.from_numpy(x).to(TORCH_DTYPES[dtype]).double().numpy()
    q_o = rnd(oracle.rotary.rotate(to_f64(d["q"]), pos, c64, s64))
    kn_o = rnd(oracle.rotary.rotate(to_f64(d["k_new"]), pos, c64, s64))
    kr, vr = oracle.rolling.append(to_f64(d["k_cache"]), to_f64(d["v_cache"]), kn_o,
                                   to_f64(d["v_new"]), s)
    # turned rows within an ulp: compare the ring within bf16 rounding of the turn
    err = np.abs(to_f64(kc) - kr)
    assert float(err.max()) <= 2.0 ** -7 * max(1.0, float(np.abs(kr).max()))
    want = oracle.rolling.decode(q_o, kr, vr, s, scale=w.sm_scale, window=W, smooth_softmax=True)
    compare(out, want, dtype, "rolling + rotary")
