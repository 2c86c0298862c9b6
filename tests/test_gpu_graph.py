"""A decode step (gqa_append_kv then gqa_decode) captured once in a HIP graph
and replayed: every replay gives the eager result bit for bit, with eager
calls on the same workspace and synchronisations between the replays.  This
is how the benchmark runs its step, so the graph path is checked the same way
as the eager one (the eager result itself is checked against the oracle).
"""

import pytest
import torch

from gpu_util import compare, make_plan, oracle_decode
from windowed_gqa_kv_amd.inputs import Workload, generate

pytestmark = pytest.mark.gpu

CASES = [
    Workload("graph", "decode", "bf16", B=4, Hq=16, Hkv=4, D=128, Lq=1, Lk=1024, window=-1,
             smooth_softmax=True, seqlens=("list", [1023, 5, 600, 300]), seed=31),
    Workload("graph", "decode", "bf16", B=2, Hq=16, Hkv=8, D=256, Lq=4, Lk=2048, window=700,
             head_sink=True, softcap=50.0, seqlens=("list", [2047, 900]), seed=32),
]


@pytest.mark.parametrize("w", CASES, ids=["d128_curr1", "d256_curr4_window_sink_softcap"])
def test_decode_step_graph_replays(gpu, w):
    d = generate(w)
    plan = make_plan(w)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq, q = d["seqlens_k"].cuda(), d["q"].cuda()
    kn, vn = d["k_new"].cuda(), d["v_new"].cuda()
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    ws = torch.zeros(plan.workspace_size(), dtype=torch.uint8, device="cuda")

    out_e = torch.empty_like(q)
    plan.append_kv(kn, vn, kc, vc, seq)
    plan.decode(q, kc, vc, seq, out_e, head_sink=sink, workspace=ws)
    torch.cuda.synchronize()
    compare(out_e, oracle_decode(w, d), w.dtype, f"eager {w}")

    # appending the same rows again rewrites the same slots with the same values
    out_g = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.append_kv(kn, vn, kc, vc, seq)
        plan.decode(q, kc, vc, seq, out_g, head_sink=sink, workspace=ws)
    torch.cuda.synchronize()

    other = torch.empty_like(q)
    for rep in range(4):
        out_g.fill_(float("nan"))
        other.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        plan.decode(q, kc, vc, seq, other, head_sink=sink, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}"
        assert torch.equal(other, out_e), f"eager call after replay {rep}"


def test_decode_steps_chained_in_one_graph(gpu):
    """Two steps (two caches) captured back to back in one graph, as the
    benchmark replays them: every replay gives each step's eager result."""
    w = CASES[0]
    d = generate(w)
    plan = make_plan(w)
    caches = [(d["k_cache"].cuda(), d["v_cache"].cuda()) for _ in range(2)]
    seq, q = d["seqlens_k"].cuda(), d["q"].cuda()
    kn, vn = d["k_new"].cuda(), d["v_new"].cuda()
    ws = torch.zeros(plan.workspace_size(), dtype=torch.uint8, device="cuda")
    out_e = torch.empty_like(q)
    plan.append_kv(kn, vn, *caches[0], seq)
    plan.decode(q, *caches[0], seq, out_e, workspace=ws)
    torch.cuda.synchronize()
    compare(out_e, oracle_decode(w, d), w.dtype, f"eager {w}")
    outs = [torch.empty_like(q) for _ in range(2)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(2):
            plan.append_kv(kn, vn, *caches[i], seq)
            plan.decode(q, *caches[i], seq, outs[i], workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], out_e), f"replay {rep}, step {i}"
