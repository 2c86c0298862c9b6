"""Helpers for the GPU tests: run a workload through the C ABI, run the same
seeded inputs through the oracle, compare.

Inputs come from windowed_gqa_kv_amd.inputs (seeded, shared by both sides);
expected values come only from the oracle.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from windowed_gqa_kv_amd import binding
from windowed_gqa_kv_amd.inputs import Workload, generate, to_f64

TOL = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3), "f16": (2e-2, 2e-3)}


def make_plan(w: Workload, **over) -> binding.Plan:
    kw = dict(dtype=w.dtype, scale=w.sm_scale, local_window_size=w.window, softcap=w.softcap,
              smooth_softmax=w.smooth_softmax, use_head_sink=w.head_sink, is_causal=w.causal,
              max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    kw.update(over)
    return binding.Plan(w.Hq, w.Hkv, w.D, **kw)


def dev(x):
    return None if x is None else x.cuda()


def gpu_prefill(w: Workload, d: dict, plan=None, layout="bhsd"):
    plan = plan or make_plan(w)
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    if layout == "bshd":
        q = q.transpose(1, 2).contiguous().view(w.B, w.Lq, w.Hq * w.D)
        k = k.transpose(1, 2).contiguous().view(w.B, w.Lk, w.Hkv * w.D)
        v = v.transpose(1, 2).contiguous().view(w.B, w.Lk, w.Hkv * w.D)
    out = plan.prefill(q, k, v, nonpad_kv_seqlen=dev(d.get("nonpad")),
                       head_sink=dev(d.get("head_sink")), layout=layout)
    torch.cuda.synchronize()
    if layout == "bshd":
        out = out.view(w.B, w.Lq, w.Hq, w.D).transpose(1, 2)
    return out


def gpu_decode(w: Workload, d: dict, plan=None):
    """append_kv then decode; returns (out, k_cache, v_cache) on the device."""
    plan = plan or make_plan(w)
    kc, vc = dev(d["k_cache"]).clone(), dev(d["v_cache"]).clone()
    seq = dev(d["seqlens_k"])
    plan.append_kv(dev(d["k_new"]), dev(d["v_new"]), kc, vc, seq)
    out = plan.decode(dev(d["q"]), kc, vc, seq, head_sink=dev(d.get("head_sink")))
    torch.cuda.synchronize()
    return out, kc, vc


def oracle_prefill(w: Workload, d: dict, rows=None, heads=None):
    """float64 oracle on the same inputs; optionally a subset of rows/heads
    (per head through the oracle's own head map on a one-head slice)."""
    sink = to_f64(d.get("head_sink"))
    nonpad = None if d.get("nonpad") is None else d["nonpad"].numpy()
    kw = dict(scale=w.sm_scale, causal=w.causal, window=w.window, softcap=w.softcap,
              smooth_softmax=w.smooth_softmax, nonpad_kv_seqlen=nonpad, rows=rows)
    if heads is None:
        return oracle.prefill(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), head_sink=sink, **kw)
    out = {}
    G = w.Hq // w.Hkv
    for h in heads:
        g = h // G
        out[h] = oracle.prefill(to_f64(d["q"][:, h:h + 1]), to_f64(d["k"][:, g:g + 1]),
                                to_f64(d["v"][:, g:g + 1]),
                                head_sink=None if sink is None else sink[h:h + 1], **kw)[:, 0]
    return out


def oracle_decode(w: Workload, d: dict):
    """Oracle append then decode.  Slots past the longest sequence are sliced
    off first: no query may see them (pinned by the oracle's stale-slot test)."""
    s = d["seqlens_k"].numpy().astype(np.int64)
    top = int(s.max()) + 1
    kc = to_f64(d["k_cache"][:, :, :top])
    vc = to_f64(d["v_cache"][:, :, :top])
    kc, vc = oracle.append_kv(kc, vc, to_f64(d["k_new"]), to_f64(d["v_new"]), s)
    return oracle.decode(to_f64(d["q"]), kc, vc, s, scale=w.sm_scale, causal=w.causal,
                         window=w.window, softcap=w.softcap, smooth_softmax=w.smooth_softmax,
                         head_sink=to_f64(d.get("head_sink")))


def compare(got, want, dtype, what=""):
    """Max-abs (and mean-abs for 16-bit types) against the float64 oracle."""
    g = got if isinstance(got, np.ndarray) else to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - want)
    max_tol, mean_tol = TOL[dtype]
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_tol, f"{what}: max-abs {mx:.3e} > {max_tol:.0e}"
    if mean_tol is not None:
        assert mn <= mean_tol, f"{what}: mean-abs {mn:.3e} > {mean_tol:.0e}"
    return mx, mn
