"""gqa_decode_noalloc (the decode whose split-KV partials and arrival
counters live in the library's static scratch array) against gqa_decode with
a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, each output bitwise equal to the workspace call's and within
the bf16 tolerances of the float64 oracle; and a call that needs more scratch
than the array holds is rejected before any launch."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import compare, make_plan, oracle_decode
from windowed_gqa_kv_amd import binding as bd
from windowed_gqa_kv_amd.inputs import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu


def _views(d, plan_w):
    q = d["q"].cuda()
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq = d["seqlens_k"].cuda()
    return q, kc, vc, seq


def _run_both(w, d, plan):
    """append once, then gqa_decode (workspace) and gqa_decode_noalloc on the
    same cache; returns both outputs."""
    q, kc, vc, seq = _views(d, w)
    plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq)
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    B, _, curr, _ = q.shape
    cap = kc.shape[2]
    ws = plan.new_workspace(q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out_ws = torch.full_like(q, float("nan"))
    out_na = torch.full_like(q, float("nan"))
    sp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    bd.check(bd.gqa_decode(plan.handle, B, curr, cap, bd.tensor_view(q), bd.tensor_view(kc),
                           bd.tensor_view(vc), bd.tensor_view(out_ws), sp(seq), sp(sink),
                           sp(ws), ws.numel(), stream))
    bd.check(bd.gqa_decode_noalloc(plan.handle, B, curr, cap, bd.tensor_view(q), bd.tensor_view(kc),
                                   bd.tensor_view(vc), bd.tensor_view(out_na), sp(seq), sp(sink),
                                   stream))
    torch.cuda.synchronize()
    return out_ws, out_na


def test_noalloc_matches_workspace_decode(gpu):
    cases = [
        # the single-token decode workload (64 row tiles), then a smaller one
        # with fewer tiles, a window, a sink and several tokens per step
        WORKLOADS[2],
        Workload("noalloc_small", "decode", "bf16", B=3, Hq=8, Hkv=2, D=128, Lq=3, Lk=700, window=200,
                 head_sink=True, seqlens=("list", [2, 350, 699]), seed=4401),
    ]
    for i, w in enumerate(cases):
        print(f"noalloc call {i}: {w}", flush=True)
        d = generate(w)
        plan = make_plan(w)
        out_ws, out_na = _run_both(w, d, plan)
        assert torch.equal(out_ws, out_na), f"call {i}: noalloc differs from the workspace decode"
        mx, mn = compare(out_na, oracle_decode(w, d), w.dtype, f"noalloc call {i}")
        print(f"noalloc call {i}: bitwise equal, max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)


def test_noalloc_rejects_oversize(gpu):
    """Head size 256 with 1024 row tiles needs more than the 16 MiB array."""
    w = Workload("noalloc_big", "decode", "bf16", B=64, Hq=16, Hkv=16, D=256, Lq=1, Lk=16,
                 window=-1, seqlens=("list", [15] * 64), seed=4402)
    plan = make_plan(w)
    q = torch.zeros(64, 16, 1, 256, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(64, 16, 16, 256, dtype=torch.bfloat16, device="cuda")
    seq = torch.full((64,), 15, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = bd.gqa_decode_noalloc(plan.handle, 64, 1, 16, bd.tensor_view(q), bd.tensor_view(kc),
                               bd.tensor_view(kc), bd.tensor_view(out),
                               ctypes.c_void_p(seq.data_ptr()), None, stream)
    assert st == bd.GQA_ERR_CAPACITY, bd.STATUS_NAMES.get(st, st)
    assert "scratch" in bd.gqa_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0  # nothing was launched
