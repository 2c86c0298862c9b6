"""Exact probes at the full workload shapes (bf16), where the output tolerance
could hide a one-key mask error.

With K = 0 every logit is 0 (and softcap(0) = 0), so every allowed key gets
weight 1/(n_i + e^{s_h}):
  * mask probe: V[j, d] = 1 iff j == probe[d]  =>  O[i, d] != 0 iff key probe[d]
    is allowed for row i, and then O[i, d] = 1 / (n_i + e^{s_h});
  * sink probe: V = 1                          =>  O[i, :] = n_i / (n_i + e^{s_h});
  * head-map probe: V[b, g] = g + 1            =>  O[b, h] = (h // G + 1) n_i / (n_i + e^{s_h}).
The allowed set and n_i come from the oracle's elementwise predicate.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import make_plan
from windowed_gqa_kv_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8  # one bf16 ulp, relative


def _counts_and_probe(q_off, Lq, valid, causal, window, probe, chunk=2048):
    """(n_i for every row, allowed(i, probe[d]) for every row and column)."""
    Lk = max(int(valid), int(np.max(probe)) + 1, 1)
    j = np.arange(Lk)
    n = np.empty(Lq, dtype=np.int64)
    hit = np.empty((Lq, len(probe)), dtype=bool)
    for r0 in range(0, Lq, chunk):
        p = q_off + np.arange(r0, min(Lq, r0 + chunk))
        n[r0:r0 + len(p)] = oracle.allowed(p[:, None], j[None, :], valid, causal, window).sum(1)
        hit[r0:r0 + len(p)] = oracle.allowed(p[:, None], np.asarray(probe)[None, :], valid,
                                             causal, window)
    return n, hit


def _sinks(w, d):
    if d is not None:
        return d.numpy().astype(np.float64)
    return np.zeros(w.Hq) if w.smooth_softmax else None


def _check_probe(got, n, hit, sink_h, scale_v=1.0, mode="mask"):
    """got: [rows, D] float64 for one (batch, head)."""
    es = 0.0 if sink_h is None else math.exp(sink_h)
    with np.errstate(divide="ignore", invalid="ignore"):
        base = np.where(n > 0, 1.0 / (n + es), 0.0)
    if mode == "mask":
        want = np.where(hit, base[:, None], 0.0)
    else:
        want = np.broadcast_to((scale_v * n * base)[:, None], got.shape)
    assert np.array_equal(got != 0, want != 0), "zero pattern differs"
    err = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert float(err[want != 0].max(initial=0.0)) <= BF16_REL


def _prefill_probe(w, mode, probe=None):
    torch.manual_seed(0)
    nonpad = None if w.nonpad is None else torch.tensor(w.nonpad, dtype=torch.int64)
    sink = torch.randn(w.Hq) if w.head_sink else None
    q = torch.randn(w.B, w.Hq, w.Lq, w.D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(w.B, w.Hkv, w.Lk, w.D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(w.B, w.Hkv, w.Lk, w.D, dtype=torch.bfloat16, device="cuda")
    if mode == "mask":
        for d_, j in enumerate(probe):
            v[:, :, j, d_] = 1.0
    elif mode == "sink":
        v.fill_(1.0)
    else:
        for g in range(w.Hkv):
            v[:, g] = g + 1
    plan = make_plan(w)
    out = plan.prefill(q, k, v, nonpad_kv_seqlen=None if nonpad is None else nonpad.cuda(),
                       head_sink=None if sink is None else sink.cuda())
    torch.cuda.synchronize()
    sinks = _sinks(w, sink)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        valid = w.Lk if nonpad is None else int(nonpad[b])
        n, hit = _counts_and_probe(w.Lk - w.Lq, w.Lq, valid, w.causal, w.window,
                                   probe if probe is not None else [0])
        heads = range(w.Hq) if w.Hq <= 32 else list(range(0, w.Hq, 7)) + [w.Hq - 1]
        for h in heads:
            got = out[b, h].double().cpu().numpy()
            s_h = None if sinks is None else sinks[h]
            _check_probe(got, n, hit, s_h, scale_v=(h // G + 1) if mode == "map" else 1.0,
                         mode="mask" if mode == "mask" else "sum")


def _mask_keys(L, extra, D, seed):
    rng = np.random.default_rng(seed)
    keys = [k for k in extra if 0 <= k < L]
    keys += rng.integers(0, L, D - len(keys)).tolist()
    return np.array(keys[:D])


@pytest.mark.parametrize("mode", ["mask", "sink", "map"])
def test_long_prefill_probes(gpu, mode):
    w = WORKLOADS[3]
    probe = _mask_keys(w.Lk, [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 4094, 4095, 4096,
                              4097, 8126, 8127, 8128, 8190, 8191], w.D, 31)
    _prefill_probe(w, mode, probe if mode == "mask" else None)


@pytest.mark.parametrize("mode", ["mask", "sink", "map"])
def test_large_gqa_prefill_probes(gpu, mode):
    w = WORKLOADS[5]
    probe = _mask_keys(w.Lk, [0, 1, 127, 128, 8190, 8191, 8192, 8193, 16383, 16384, 24574,
                              24575, 24576, 24577, 32703, 32704, 32766, 32767], w.D, 51)
    _prefill_probe(w, mode, probe if mode == "mask" else None)


@pytest.mark.parametrize("mode", ["mask", "sink", "map"])
@pytest.mark.parametrize("D", [32, 256])
def test_prefill_probes_other_head_sizes(gpu, mode, D):
    """Head sizes 32 and 256 on the matrix-core prefill: a 4096-key prompt
    with a window, a sink and (head size 32) padded keys."""
    from windowed_gqa_kv_amd.inputs import Workload
    if D == 256:
        w = Workload("probe256", "prefill", "bf16", B=1, Hq=16, Hkv=8, D=256, Lq=4096, Lk=4096, window=1000,
                     head_sink=True, seed=0)
    else:
        w = Workload("probe32", "prefill", "bf16", B=2, Hq=8, Hkv=2, D=32, Lq=4096, Lk=4096, window=700,
                     head_sink=True, nonpad=(4096, 3000), seed=0)
    probe = _mask_keys(w.Lk, [0, 1, 63, 64, 699, 700, 999, 1000, 2999, 3000, 3001, 4094, 4095], D, 7 + D)
    _prefill_probe(w, mode, probe if mode == "mask" else None)


def _decode_probe(w, seqlens, mode, probe=None):
    torch.manual_seed(1)
    B, curr, cap = w.B, w.Lq, w.Lk
    sink = torch.randn(w.Hq) if w.head_sink else None
    seq = torch.tensor(seqlens, dtype=torch.int32)
    total = seq.numpy().astype(np.int64) + 1
    q = torch.randn(B, w.Hq, curr, w.D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, w.Hkv, cap, w.D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(B, w.Hkv, cap, w.D, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(B, w.Hkv, curr, w.D, dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros(B, w.Hkv, curr, w.D, dtype=torch.bfloat16, device="cuda")
    if mode == "mask":
        for b in range(B):
            for d_, j in enumerate(probe[b]):
                t = j - (total[b] - curr)
                if 0 <= t < curr:
                    vn[b, :, t, d_] = 1.0   # the probe key arrives through append_kv
                else:
                    vc[b, :, j, d_] = 1.0
    elif mode == "sink":
        vc.fill_(1.0)
        vn.fill_(1.0)
    else:
        for g in range(w.Hkv):
            vc[:, g] = g + 1
            vn[:, g] = g + 1
    # stale slots hold garbage that must never be read
    for b in range(B):
        vc[b, :, total[b]:] = float("nan")
        kc[b, :, total[b]:] = float("nan")
    plan = make_plan(w)
    seq_d = seq.cuda()
    plan.append_kv(kn, vn, kc, vc, seq_d)
    out = plan.decode(q, kc, vc, seq_d, head_sink=None if sink is None else sink.cuda())
    torch.cuda.synchronize()
    sinks = _sinks(w, sink)
    G = w.Hq // w.Hkv
    for b in range(B):
        n, hit = _counts_and_probe(int(total[b]) - curr, curr, int(total[b]), w.causal, w.window,
                                   probe[b] if probe is not None else [0])
        for h in range(w.Hq):
            got = out[b, h].double().cpu().numpy()
            s_h = None if sinks is None else sinks[h]
            _check_probe(got, n, hit, s_h, scale_v=(h // G + 1) if mode == "map" else 1.0,
                         mode="mask" if mode == "mask" else "sum")


@pytest.mark.parametrize("mode", ["mask", "sink", "map"])
def test_single_token_decode_probes(gpu, mode):
    w = WORKLOADS[2]
    seqlens = [1024, 1500, 2047, 2048, 2049, 3000, 4000, 4095]
    probe = None
    if mode == "mask":
        probe = []
        for b, s in enumerate(seqlens):
            extra = [0, 1, 255, 256, 257, s - 1, s, s + 1, s + 2, 4095]
            probe.append(_mask_keys(4096, extra, w.D, 70 + b))
    _decode_probe(w, seqlens, mode, probe)


@pytest.mark.parametrize("mode", ["mask", "sink", "map"])
def test_spec_decode_probes(gpu, mode):
    w = WORKLOADS[4]
    seqlens = [16387, 16387, 5000, 32767]
    probe = None
    if mode == "mask":
        probe = []
        for b, s in enumerate(seqlens):
            extra = [0, s - 4098, s - 4097, s - 4096, s - 4095, s - 4094, s - 3, s - 2, s - 1, s,
                     s + 1, 32767]
            probe.append(_mask_keys(32768, extra, w.D, 90 + b))
    _decode_probe(w, seqlens, mode, probe)
