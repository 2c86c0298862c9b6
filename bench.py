"""Benchmark of the windowed GQA hot path on one MI355X.

Default workload: single-token decode, bf16, B=8, Hq=32, Hkv=8, D=128, KV
capacity 4096, seqlens_k ~ integers[1024, 4096), smooth_softmax (zero sink),
window off.  One step = the whole decode path for one batch:
gqa_append_decode, one launch that puts the new token's K/V into the cache
and runs the split-KV attention with the merge of the splits (the same step
as two launches, gqa_append_kv then gqa_decode, is timed beside it).  Inputs are resident in HBM before
timing starts.  Every step works on a different replica of the KV cache (R
replicas, >= 1 GiB in total), so a step cannot be served from the 256 MB
Infinity Cache left warm by the previous one.

Prints ONE JSON line.  `value` = algorithmic bytes of the step (K/V rows of
the kept key range, Q, O, and the appended rows) / wall time per step, the
steps being replayed from HIP graphs that hold one step per cache replica in
turn (captured once, as consecutive layers of a serving loop would run);
the eager per-step time is reported too.
`roofline` is for the dominant kernel (the step's one launch): its average
duration is timed with HIP events on the stream it runs on, around graphs of
back-to-back launches (one per cache replica); events around each eager
launch, which also count its dispatch latency, are reported beside it, and so
is the decode kernel alone (gqa_decode).  `cpu_baseline` times the float64 oracle on
this host (the oracle as it stands, on a bounded number of full decode
steps).  `extra` reports the prompt workloads (TFLOP/s against the bf16 MFMA
peak) and the speculative-decode workload the same way; `rotary` times the
rotary embedding of the long prompt's Q and K (GB/s against HBM) and a decode
step's append with rotary beside the plain append; `rolling` times the
speculative-decode workload against a rolling cache of W + curr - 1 slots;
`masks` times the long prompt through the masked matrix-core prefill with an
all-True and block-sparse boolean masks (16x64 and 128x64 blocks), an
additive one and one with softcap, beside the unmasked prefill; `fp8` times
the headline decode on FP8 (E4M3) caches, and on INT8 caches with per-KV-head
scales; `peaks_measured` reports the dense
bf16 MFMA rate and shader clock measured on the device and a 1 GiB copy's
rate, for context (fractions stay against the published peaks).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
       [--no-cpu-baseline] [--workload NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "prefill TFLOP/s (%MFMA peak); decode KV-cache GB/s (%HBM peak), 1 MI355X"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_1tok_bf16")
    ap.add_argument("--replicas", type=int, default=0, help="KV replicas (0 = enough for 1 GiB)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (the reference kernel that "
                         "scales the FETCH_SIZE/WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: float):
    """10 device-to-device copies of a known size, for counter calibration."""
    import torch
    n = int(mib * (1 << 20))
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(10):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "copies": 10}), flush=True)


def _traffic(kernel: str, workload: str, src_files):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    from windowed_gqa_kv_amd.profiling import src_hash
    rec = table.get(f"{kernel}/{workload}")
    if not rec or rec.get("src_hash") != src_hash(src_files):
        return None
    return rec.get("bytes_per_launch")


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def bench_decode(w, steps, warmup, replicas):
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import generate

    d = generate(w)
    plan = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, scale=w.sm_scale, local_window_size=w.window,
                        softcap=w.softcap, smooth_softmax=w.smooth_softmax, use_head_sink=w.head_sink,
                        is_causal=w.causal, max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    kv_bytes = 2 * d["k_cache"].numel() * d["k_cache"].element_size()
    R = replicas or max(2, -(-(1 << 30) // kv_bytes))
    kc0, vc0 = d["k_cache"].cuda(), d["v_cache"].cuda()
    caches = [(kc0.clone(), vc0.clone()) for _ in range(R)]
    del kc0, vc0
    q = d["q"].cuda()
    kn, vn = d["k_new"].cuda(), d["v_new"].cuda()
    seq = d["seqlens_k"].cuda()
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(16, plan.workspace_size()), dtype=torch.uint8, device="cuda")

    def step(i, ev=None):
        # one decode step: the new token's K/V into the cache and the
        # attention, one launch (gqa_append_decode)
        kc, vc = caches[i % R]
        if ev is not None:
            ev[0].record()
        plan.append_decode(q, kn, vn, kc, vc, seq, out, head_sink=sink, workspace=ws)
        if ev is not None:
            ev[1].record()

    def step_two_launches(i):
        kc, vc = caches[i % R]
        plan.append_kv(kn, vn, kc, vc, seq)
        plan.decode(q, kc, vc, seq, out, head_sink=sink, workspace=ws)

    # Eager steps: warm-up, then each launch timed with HIP events on the
    # stream it runs on (dispatch latency included).
    for i in range(warmup):
        step(i)
    evs = _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms_events_each = sum(a.elapsed_time(b) for a, b in evs) / steps
    eager_ms = (t1 - t0) * 1000.0 / steps

    # The step as a serving loop runs it, from HIP graphs: one graph holds R
    # consecutive steps (one per cache replica, as consecutive layers would
    # run), another one step per replica; K steps are floor(K / R) replays of
    # the first and K mod R of the second, so the host's per-launch work is
    # out of the step.
    def graphs_of(fn):
        chain = torch.cuda.CUDAGraph()
        with torch.cuda.graph(chain):
            for r in range(R):
                fn(r)
        single = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(r)
            single.append(g)
        return chain, single

    def time_steps(chain, single):
        for i in range(max(1, warmup // R)):
            chain.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps // R):
            chain.replay()
        for i in range(steps % R):
            single[i].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / steps

    chain, single = graphs_of(step)
    ms = time_steps(chain, single)
    del chain, single
    chain, single = graphs_of(step_two_launches)
    ms_two = time_steps(chain, single)
    del chain, single

    # Average kernel durations for the roofline: launches back to back (one
    # per replica, from a graph), between two HIP events on the stream they
    # run on -- the fused step's kernel, and the decode alone.
    def b2b(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(R):
                fn(r)
        g.replay()
        nrep = max(1, steps // R)
        e0, e1 = _events(1)[0]
        torch.cuda.synchronize()
        e0.record()
        for i in range(nrep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (nrep * R)

    fused_ms = b2b(step)
    dec_ms = b2b(lambda r: plan.decode(q, caches[r][0], caches[r][1], seq, out, head_sink=sink, workspace=ws))
    s = d["seqlens_k"].numpy()
    stream = kv_stream_ceiling(w, s, caches, b2b) if w.D in (128, 256) and w.dtype != "f32" else None
    dec_bytes = work.decode_bytes(s, w.Lq, w.Hq, w.Hkv, w.D, w.dtype, w.causal, w.window)
    app_bytes = work.append_bytes(w.B, w.Hkv, w.Lq, w.D, w.dtype)
    return dict(ms_per_step=ms, two_launch_ms_per_step=ms_two, eager_ms_per_step=eager_ms,
                step_bytes=dec_bytes + app_bytes, kernel_ms=fused_ms, kernel_ms_events_each=step_ms_events_each,
                decode_only_ms=dec_ms, decode_bytes=dec_bytes, replicas=R, inputs=d, stream=stream)


def _ceiling(st):
    rate = st["bytes"] / (st["kernel_ms"] / 1e3) / 1e9
    return {"kernel": "kv_stream_probe_kernel (the decode's K/V units through its LDS-DMA loading scheme, "
                      "no attention work)",
            "units": st["units"], "grid": st["grid"], "kernel_ms": round(st["kernel_ms"], 5),
            "bytes_per_launch": st["bytes"], "achieved": round(rate, 2), "frac": round(rate / PEAK_HBM_GBS, 4)}


def kv_stream_ceiling(w, seqlens, caches, b2b):
    """The decode's own K/V units (16 keys from each tile's first allowed key
    on, K and V) streamed by the library's probe through the decode's
    loading scheme, with no attention work, at the decode's workgroups per CU
    (two at head size 128, one at 256), timed like the decode (back to back
    over the cache replicas): the rate this loading scheme reaches on these
    bytes."""
    import ctypes

    import numpy as np
    import torch
    from windowed_gqa_kv_amd import binding

    row_bytes = 2 * w.D
    offs = []
    for b in range(w.B):
        valid = int(seqlens[b]) + 1
        q_off = valid - w.Lq
        lo = 0 if w.window < 0 else max(0, q_off - w.window + 1)
        n_units = (valid - 1 - lo) // 16 + 1
        for g in range(w.Hkv):
            base = (b * w.Hkv + g) * w.Lk + lo
            offs.extend((base + 16 * u) * row_bytes for u in range(n_units))
    off = torch.tensor(np.array(offs, dtype=np.int64), device="cuda")
    sink = torch.zeros(1, device="cuda")
    kv_bytes = caches[0][0].numel() * caches[0][0].element_size()
    grid = (2 if w.D == 128 else 1) * torch.cuda.get_device_properties(0).multi_processor_count
    U = len(offs)

    def probe(r):
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = binding.gqa_probe_kv_stream(grid, row_bytes, ctypes.c_void_p(caches[r][0].data_ptr()),
                                         ctypes.c_void_p(caches[r][1].data_ptr()), kv_bytes,
                                         ctypes.c_void_p(off.data_ptr()), U, ctypes.c_void_p(sink.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"K/V stream probe failed ({rc})")

    ms = b2b(probe)
    return dict(kernel_ms=ms, units=U, bytes=U * 2 * 16 * row_bytes, grid=grid)


def bench_prefill(w, steps, warmup, d=None):
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import generate

    d = d if d is not None else generate(w)
    plan = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, scale=w.sm_scale, local_window_size=w.window,
                        softcap=w.softcap, smooth_softmax=w.smooth_softmax, use_head_sink=w.head_sink,
                        is_causal=w.causal, max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    q, k, v = d["q"].cuda(), d["k"].cuda(), d["v"].cuda()
    nonpad = None if d["nonpad"] is None else d["nonpad"].cuda()
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    out = torch.empty_like(q)
    for _ in range(warmup):
        plan.prefill(q, k, v, out, nonpad_kv_seqlen=nonpad, head_sink=sink)
    evs = _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record()
        plan.prefill(q, k, v, out, nonpad_kv_seqlen=nonpad, head_sink=sink)
        evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flops = work.prefill_flops(w.B, w.Hq, w.D, w.Lq, w.Lk, w.causal, w.window, w.nonpad)
    kms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return dict(ms_per_step=(t1 - t0) * 1000.0 / steps, flops=flops, kernel_ms=kms)


def bench_rotary(steps, warmup):
    """Rotary embedding: the long prompt's Q and K turned by gqa_apply_rotary
    (HIP events around each launch; the inputs rotate over 8 replicas, 640 MiB,
    so that no launch reads them from the Infinity Cache), and one decode
    step's gqa_append_kv_rotary
    against the plain gqa_append_kv (graphs of `steps` back-to-back launches,
    HIP events around the replays)."""
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import WORKLOADS, generate, rotary_tables

    res = {}
    wp = WORKLOADS[3]
    d = generate(wp)
    plan = binding.Plan(wp.Hq, wp.Hkv, wp.D, dtype=wp.dtype, local_window_size=wp.window,
                        max_batch=wp.B, max_q_len=wp.Lq, max_kv_len=wp.Lk)
    cos, sin = (t.cuda() for t in rotary_tables(wp.Lk, wp.D))
    R = 8
    q0, k0 = d["q"].cuda(), d["k"].cuda()
    qs, ks = [q0.clone() for _ in range(R)], [k0.clone() for _ in range(R)]
    qo, ko = torch.empty_like(q0), torch.empty_like(k0)
    del d, q0, k0
    for i in range(warmup):
        plan.apply_rotary(qs[i % R], wp.Lk - wp.Lq, cos, sin, qo)
        plan.apply_rotary(ks[i % R], 0, cos, sin, ko)
    evq, evk = _events(steps), _events(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        evq[i][0].record()
        plan.apply_rotary(qs[i % R], wp.Lk - wp.Lq, cos, sin, qo)
        evq[i][1].record()
        evk[i][0].record()
        plan.apply_rotary(ks[(i + R // 2) % R], 0, cos, sin, ko)
        evk[i][1].record()
    torch.cuda.synchronize()
    ms_q = sum(a.elapsed_time(b) for a, b in evq) / steps
    ms_k = sum(a.elapsed_time(b) for a, b in evk) / steps
    bq = work.rotary_bytes(wp.B * wp.Hq * wp.Lq, wp.D, wp.dtype, wp.Lq)
    bk = work.rotary_bytes(wp.B * wp.Hkv * wp.Lk, wp.D, wp.dtype, wp.Lk)
    res["prompt"] = {"workload": wp.name, "q_ms": round(ms_q, 5), "k_ms": round(ms_k, 5),
                     "bytes": bq + bk, "achieved": round((bq + bk) / ((ms_q + ms_k) / 1e3) / 1e9, 2),
                     "unit": "GB/s"}
    res["prompt"]["frac"] = round(res["prompt"]["achieved"] / PEAK_HBM_GBS, 4)
    # the prompt's attention with Q turned inside the prefill
    # (gqa_prefill_rotary, K turned once beforehand) against the turn as its
    # own pass followed by gqa_prefill; Q rotates over the same 8 replicas
    v0 = torch.empty_like(ks[0]).normal_().mul_(0.5)
    out = torch.empty_like(qo)
    ev2 = {"prefill_rotary": _events(steps), "apply_rotary_q_then_prefill": _events(steps)}
    for i in range(2):
        plan.prefill_rotary(qs[i], ko, v0, cos, sin, out)
        plan.apply_rotary(qs[i], 0, cos, sin, qo)
    torch.cuda.synchronize()
    for i in range(steps):
        a, b = ev2["prefill_rotary"][i]
        a.record()
        plan.prefill_rotary(qs[i % R], ko, v0, cos, sin, out)
        b.record()
        a, b = ev2["apply_rotary_q_then_prefill"][i]
        a.record()
        plan.apply_rotary(qs[(i + R // 2) % R], 0, cos, sin, qo)
        plan.prefill(qo, ko, v0, out)
        b.record()
    torch.cuda.synchronize()
    res["prompt_attention"] = {name: round(sorted(x.elapsed_time(y) for x, y in ev)[len(ev) // 2], 5)
                               for name, ev in ev2.items()}
    res["prompt_attention"]["unit"] = "ms (median of events around each, Q cold)"
    del qs, ks, qo, ko, v0, out
    torch.cuda.empty_cache()

    wd = WORKLOADS[2]
    d = generate(wd)
    plan = binding.Plan(wd.Hq, wd.Hkv, wd.D, dtype=wd.dtype, smooth_softmax=wd.smooth_softmax,
                        max_batch=wd.B, max_q_len=wd.Lq, max_kv_len=wd.Lk)
    cos, sin = (t.cuda() for t in rotary_tables(wd.Lk, wd.D))
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    q, kn, vn, seq = d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), d["seqlens_k"].cuda()
    q_rot = torch.empty_like(q)
    calls = {"append_kv": lambda: plan.append_kv(kn, vn, kc, vc, seq),
             "append_kv_rotary": lambda: plan.append_kv_rotary(q, kn, vn, kc, vc, seq, cos, sin, q_rot)}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        ev = _events(5)
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        res[name + "_us"] = round(min(a.elapsed_time(b) for a, b in ev) * 1e3 / steps, 3)
    res["decode_step_workload"] = wd.name
    res["append_kv_rotary_bytes"] = work.append_rotary_bytes(wd.B, wd.Hq, wd.Hkv, wd.Lq, wd.D, wd.dtype)
    return res


def bench_rolling(reps):
    """The speculative-decode workload (window 4096, 4 new tokens on a past of
    16384) against a rolling cache of W + curr - 1 = 4099 slots instead of
    the 32768-slot linear cache: the same keys are read, from ring slots.
    Graphs of back-to-back decodes over 8 ring replicas (1 GiB), HIP events
    around the replays."""
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import WORKLOADS, generate

    w = WORKLOADS[4]
    d = generate(w)
    C = w.window + w.Lq - 1
    plan = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, scale=w.sm_scale, local_window_size=w.window,
                        softcap=w.softcap, smooth_softmax=w.smooth_softmax, use_head_sink=w.head_sink,
                        is_causal=w.causal, rolling_cache=True, max_batch=w.B, max_q_len=w.Lq,
                        max_kv_len=C)
    seq = d["seqlens_k"]
    top = int(seq.max()) + 1
    # ring slot p mod C holds the cache row of position p, for the last C positions
    pos = torch.arange(top - C, top)
    slots = pos % C
    ring_k = torch.empty(w.B, w.Hkv, C, w.D, dtype=d["k_cache"].dtype)
    ring_v = torch.empty_like(ring_k)
    ring_k[:, :, slots] = d["k_cache"][:, :, pos]
    ring_v[:, :, slots] = d["v_cache"][:, :, pos]
    R = 8
    rk, rv = ring_k.cuda(), ring_v.cuda()
    rings = [(rk.clone(), rv.clone()) for _ in range(R)]
    del rk, rv, ring_k, ring_v
    q, seq_d = d["q"].cuda(), seq.cuda()
    kn, vn = d["k_new"].cuda(), d["v_new"].cuda()
    sink = None if d["head_sink"] is None else d["head_sink"].cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(16, plan.workspace_size()), dtype=torch.uint8, device="cuda")
    for kc, vc in rings:
        plan.append_kv(kn, vn, kc, vc, seq_d)
        plan.decode(q, kc, vc, seq_d, out, head_sink=sink, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for kc, vc in rings:
            plan.decode(q, kc, vc, seq_d, out, head_sink=sink, workspace=ws)
    g.replay()
    torch.cuda.synchronize()
    ev = _events(reps)
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / (reps * R)
    b = work.decode_bytes(seq.numpy().astype("int64"), w.Lq, w.Hq, w.Hkv, w.D, w.dtype, w.causal, w.window)
    return {"workload": w.name, "ring_slots": C, "linear_capacity": w.Lk, "kernel_ms": round(ms, 5),
            "achieved": round(b / (ms / 1e3) / 1e9, 2), "unit": "GB/s",
            "frac": round(b / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_masks(steps):
    """The long prompt through gqa_prefill_masked with a boolean [1, 1, Lq, Lk]
    mask (the matrix-core prefill, reading the mask bytes one tile ahead): an
    all-True mask (every pair of the band evaluated) and a block-sparse one
    (about half of the 64-key blocks of every 16-row group cleared; a wave
    skips a tile its 32 rows all lose); and the same block-sparse mask as an
    additive 0 / -inf mask, evaluated in full; and the block-sparse boolean
    mask again with a softcap of 50 on the logits.  FLOPs are 4*D per kept
    pair of band and mask."""
    import numpy as np
    import torch
    from windowed_gqa_kv_amd import binding
    from windowed_gqa_kv_amd.inputs import WORKLOADS, generate

    w = WORKLOADS[3]
    d = generate(w)
    plan = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, local_window_size=w.window,
                        max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    capped = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, local_window_size=w.window, softcap=50.0,
                          max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    q, k, v = d["q"].cuda(), d["k"].cuda(), d["v"].cuda()
    out = torch.empty_like(q)
    del d
    i = (w.Lk - w.Lq) + np.arange(w.Lq)[:, None]
    j = np.arange(w.Lk)[None, :]
    band = (j <= i) & (i - j < w.window)
    rng = np.random.default_rng(5)
    keep = rng.random(((w.Lq + 15) // 16, (w.Lk + 63) // 64)) < 0.5
    sparse = np.repeat(np.repeat(keep, 16, 0), 64, 1)[:w.Lq, :w.Lk]
    keep128 = rng.random(((w.Lq + 127) // 128, (w.Lk + 63) // 64)) < 0.5
    sparse128 = np.repeat(np.repeat(keep128, 128, 0), 64, 1)[:w.Lq, :w.Lk]
    res = {"workload": w.name}
    add = np.where(sparse, 0.0, -np.inf).astype(np.float32)
    out0 = torch.empty_like(q)
    plan.prefill(q, k, v, out0)
    ev0 = _events(steps)
    torch.cuda.synchronize()
    for a, b in ev0:
        a.record()
        plan.prefill(q, k, v, out0)
        b.record()
    torch.cuda.synchronize()
    res["unmasked_kernel_ms"] = round(sum(a.elapsed_time(b) for a, b in ev0) / steps, 4)
    del out0
    for name, m, p in (("all_true", np.ones((w.Lq, w.Lk), bool), plan), ("block_sparse", sparse, plan),
                       ("block_sparse_128x64", sparse128, plan),
                       ("block_sparse_additive", add, plan), ("block_sparse_softcap50", sparse, capped)):
        md = torch.from_numpy(m)[None, None].cuda()
        m = m if m.dtype == bool else m > -np.inf
        pairs = int((band & m).sum()) * w.B * w.Hq
        p.prefill(q, k, v, out, mask=md)
        evs = _events(steps)
        torch.cuda.synchronize()
        for a, b in evs:
            a.record()
            p.prefill(q, k, v, out, mask=md)
            b.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / steps
        tf = 4 * w.D * pairs / (ms / 1e3) / 1e12
        res[name] = {"kernel": "prefill_mfma_kernel",
                     "kernel_ms": round(ms, 4), "kept_pairs": pairs, "achieved": round(tf, 2),
                     "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del md
    del q, k, v, out
    torch.cuda.empty_cache()
    # the headline decode with a random boolean mask over [B, Hq, 1, capacity]
    # (90% of the keys kept), against the same launches without a mask: eager
    # launches, HIP events around each
    wd = WORKLOADS[2]
    d = generate(wd)
    plan = binding.Plan(wd.Hq, wd.Hkv, wd.D, dtype=wd.dtype, smooth_softmax=wd.smooth_softmax,
                        max_batch=wd.B, max_q_len=wd.Lq, max_kv_len=wd.Lk)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    q, seq = d["q"].cuda(), d["seqlens_k"].cuda()
    out = torch.empty_like(q)
    ws = plan.new_workspace()
    md = torch.from_numpy(np.random.default_rng(12).random((wd.B, wd.Hq, 1, wd.Lk)) < 0.9).cuda()
    times = {}
    for name, m in (("decode_unmasked", None), ("decode_bool_mask", md)):
        for _ in range(5):
            plan.decode(q, kc, vc, seq, out, workspace=ws, mask=m)
        evs = _events(steps * 10)
        torch.cuda.synchronize()
        for a, b in evs:
            a.record()
            plan.decode(q, kc, vc, seq, out, workspace=ws, mask=m)
            b.record()
        torch.cuda.synchronize()
        times[name] = round(sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2] * 1e3, 2)
    res["decode"] = {"workload": wd.name, "kernel": "decode_kernel", "median_us_per_eager_launch": times,
                     "note": "warm cache (one replica); events around each eager launch"}
    return res


def bench_fp8(reps):
    """The headline decode on FP8 (E4M3) caches (gqa_decode_fp8): graphs of
    back-to-back decodes over 16 cache replicas (1 GiB), HIP events around the
    replays.  Bytes: the K/V rows at one byte per element, Q and O.  The same
    graphs again through gqa_decode_fp8_masked with a random boolean
    [B, Hq, 1, capacity] mask (90% of the keys kept)."""
    import numpy as np
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import WORKLOADS, generate

    w = WORKLOADS[2]
    d = generate(w)
    ks = vs = 0.03
    plan = binding.Plan(w.Hq, w.Hkv, w.D, dtype=w.dtype, smooth_softmax=w.smooth_softmax,
                        max_batch=w.B, max_q_len=w.Lq, max_kv_len=w.Lk)
    kc0 = (d["k_cache"].float() / ks).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    vc0 = (d["v_cache"].float() / vs).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    R = 16
    caches = [(kc0.clone(), vc0.clone()) for _ in range(R)]
    del kc0, vc0
    q, seq = d["q"].cuda(), d["seqlens_k"].cuda()
    kn, vn = d["k_new"].cuda(), d["v_new"].cuda()
    out = torch.empty_like(q)
    ws = plan.new_workspace()
    for kc, vc in caches:
        plan.append_kv_fp8(kn, vn, kc, vc, seq, ks, vs)
        plan.decode_fp8(q, kc, vc, seq, ks, vs, out, workspace=ws)
    torch.cuda.synchronize()
    md = torch.from_numpy(np.random.default_rng(12).random((w.B, w.Hq, 1, w.Lk)) < 0.9).cuda()
    times = []
    for mask in (None, md):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for kc, vc in caches:
                plan.decode_fp8(q, kc, vc, seq, ks, vs, out, workspace=ws, mask=mask)
        g.replay()
        torch.cuda.synchronize()
        ev = _events(reps)
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        times.append(sum(a.elapsed_time(b) for a, b in ev) / (reps * R))
        del g
    ms, ms_masked = times
    del caches
    # the same decode on INT8 caches with per-KV-head scales
    ksc = torch.full((w.Hkv,), 0.03, device="cuda")
    ic0 = torch.clamp(torch.round(d["k_cache"].float() / 0.03), -127, 127).to(torch.int8).cuda()
    iv0 = torch.clamp(torch.round(d["v_cache"].float() / 0.03), -127, 127).to(torch.int8).cuda()
    icaches = [(ic0.clone(), iv0.clone()) for _ in range(R)]
    del ic0, iv0
    for kc, vc in icaches:
        plan.append_kv_int8(kn, vn, kc, vc, seq, ksc, ksc)
        plan.decode_int8(q, kc, vc, seq, ksc, ksc, out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for kc, vc in icaches:
            plan.decode_int8(q, kc, vc, seq, ksc, ksc, out, workspace=ws)
    g.replay()
    torch.cuda.synchronize()
    ev = _events(reps)
    for a, b_ in ev:
        a.record()
        g.replay()
        b_.record()
    torch.cuda.synchronize()
    ms_i8 = sum(a.elapsed_time(b_) for a, b_ in ev) / (reps * R)
    del g, icaches
    s = d["seqlens_k"].numpy().astype("int64")
    b = work.decode_bytes(s, w.Lq, w.Hq, w.Hkv, w.D, w.dtype, w.causal, w.window, kv_dtype="fp8")
    return {"workload": w.name, "kernel": "decode_kernel (FP8 caches)", "kernel_ms": round(ms, 5),
            "bytes_per_launch": b, "achieved": round(b / (ms / 1e3) / 1e9, 2), "unit": "GB/s",
            "frac": round(b / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "bool_mask_kernel_ms": round(ms_masked, 5),
            "int8": {"kernel": "decode_kernel (INT8 caches, per-KV-head scales)", "kernel_ms": round(ms_i8, 5),
                     "bytes_per_launch": b, "achieved": round(b / (ms_i8 / 1e3) / 1e9, 2),
                     "frac": round(b / (ms_i8 / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}


def peaks_measured():
    """Context for the fractions (which stay against the published peaks):
    the dense bf16 matrix rate and the shader clock measured on this device
    by the library's probe (back-to-back register-operand MFMAs, shader-clock
    and 100 MHz stamps per wave), and a plain 1 GiB device copy's rate."""
    import ctypes

    import numpy as np
    import torch
    from windowed_gqa_kv_amd import binding

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * cus, 4000
    stamps = torch.zeros(blocks * 4 * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks * 4, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sp, kp = ctypes.c_void_p(stamps.data_ptr()), ctypes.c_void_p(sink.data_ptr())
    binding.check(0 if binding.gqa_probe_mfma_peak(blocks, 200, sp, kp, stream) == 0 else 4)
    best = None
    for _ in range(3):
        e0, e1 = _events(1)[0]
        e0.record()
        rc = binding.gqa_probe_mfma_peak(blocks, iters, sp, kp, stream)
        e1.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError("MFMA probe launch failed")
        ms = e0.elapsed_time(e1)
        st = stamps.view(-1, 4).cpu().numpy().astype(np.float64)
        clk = float(np.median((st[:, 1] - st[:, 0]) / ((st[:, 3] - st[:, 2]) / 1e8)))
        if best is None or ms < best[0]:
            best = (ms, clk)
    ms, clk = best
    flops = blocks * 4 * iters * 8 * 32768
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    y.copy_(x)
    ev = _events(5)
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        y.copy_(x)
        b.record()
    torch.cuda.synchronize()
    cms = min(a.elapsed_time(b) for a, b in ev)
    del x, y
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "shader_clock_ghz": round(clk / 1e9, 3),
            "dense_bf16_peak_at_that_clock_tflops": round(cus * 4 * 1024 * clk / 1e12, 1),
            "published_peaks": {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS},
            "copy_1gib_gbs": round(2 * (1 << 30) / (cms / 1e3) / 1e9, 1),
            "note": "fractions are against the published peaks; these are measured on this device for context"}


def bench_prefill_d256(steps):
    """A prompt at head size 256 (the speculative-decode workload's model:
    Hq 16, Hkv 8, sink, softcap 50) of 8192 tokens with a 4096-key window, on
    the matrix-core prefill."""
    import torch
    from windowed_gqa_kv_amd import binding, work
    from windowed_gqa_kv_amd.inputs import Workload, generate

    w = Workload("prefill_d256_bf16", "prefill", "bf16", B=1, Hq=16, Hkv=8, D=256, Lq=8192, Lk=8192,
                 window=4096, head_sink=True, softcap=50.0, value_scale=0.5, seed=1006)
    d = generate(w)
    r = bench_prefill(w, steps, 3, d)
    tf = r["flops"] / (r["kernel_ms"] / 1e3) / 1e12
    return {"workload": w.name, "config": {"B": 1, "Hq": 16, "Hkv": 8, "D": 256, "L": 8192, "window": 4096,
                                           "head_sink": True, "softcap": 50.0},
            "kernel_ms": round(r["kernel_ms"], 5), "achieved": round(tf, 2), "unit": "TFLOP/s",
            "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(w, d, budget_s=12.0):
    """The float64 oracle on full decode steps of the same workload, repeated
    until ~budget_s of CPU time; reported in the same unit (GB/s)."""
    import numpy as np
    import oracle
    from windowed_gqa_kv_amd import work
    from windowed_gqa_kv_amd.inputs import to_f64

    s = d["seqlens_k"].numpy().astype(np.int64)
    top = int(s.max()) + 1
    kc = to_f64(d["k_cache"][:, :, :top])
    vc = to_f64(d["v_cache"][:, :, :top])
    kc, vc = oracle.append_kv(kc, vc, to_f64(d["k_new"]), to_f64(d["v_new"]), s)
    q = to_f64(d["q"])
    sink = to_f64(d["head_sink"])
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode(q, kc, vc, s, scale=w.sm_scale, causal=w.causal, window=w.window,
                      softcap=w.softcap, smooth_softmax=w.smooth_softmax, head_sink=sink)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    b = work.decode_bytes(s, w.Lq, w.Hq, w.Hkv, w.D, w.dtype, w.causal, w.window)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{n} full decode steps of the same workload (append + decode, float64 "
                      f"materialized oracle, {dt * 1e3:.1f} ms each)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the attention path has no multi-GPU mode "
              f"(requested --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    from windowed_gqa_kv_amd import binding
    from windowed_gqa_kv_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    binding.load()
    byname = {w.name: w for w in WORKLOADS.values()}
    w = byname[args.workload]
    if w.kind != "decode":
        print("the headline workload must be a decode workload", file=sys.stderr)
        sys.exit(2)

    r = bench_decode(w, args.steps, args.warmup, args.replicas)
    value = r["step_bytes"] / (r["ms_per_step"] / 1e3) / 1e9
    achieved = r["step_bytes"] / (r["kernel_ms"] / 1e3) / 1e9
    dec_only = r["decode_bytes"] / (r["decode_only_ms"] / 1e3) / 1e9
    dec_src = ["decode_mfma.hip", "common.h", "kernels.h"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1); KV cache rotated over "
                f"{r['replicas']} replicas so no step reads a warm Infinity Cache)",
        "step": f"gqa_append_decode (the new token's K/V into the cache and the attention, one launch); "
                f"timed from HIP graphs of {r['replicas']} consecutive steps (one per cache replica); "
                f"eager launches take {r['eager_ms_per_step'] * 1e3:.1f} us per step; as two launches "
                f"(gqa_append_kv, gqa_decode) a step takes {r['two_launch_ms_per_step'] * 1e3:.1f} us",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "curr": w.Lq, "kv_capacity": w.Lk, "window": w.window,
                   "seqlens_k": [int(x) for x in r["inputs"]["seqlens_k"].numpy()],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": "decode_kernel (gqa_append_decode: the step's append, the split-KV stream and "
                               "the fused combine)",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": _traffic("append_decode", w.name, dec_src),
                     "kernel_ms": round(r["kernel_ms"], 5), "bytes_per_launch": r["step_bytes"],
                     "timing": f"HIP events around {r['replicas']}-launch graphs of back-to-back launches; "
                               f"events around each eager launch read {r['kernel_ms_events_each'] * 1e3:.1f} us",
                     "decode_only": {"kernel": "decode_kernel (gqa_decode)", "kernel_ms": round(r["decode_only_ms"], 5),
                                     "bytes_per_launch": r["decode_bytes"], "achieved": round(dec_only, 2),
                                     "frac": round(dec_only / PEAK_HBM_GBS, 4),
                                     "traffic": _traffic("decode", w.name, dec_src)}},
    }
    if r["stream"] is not None:
        line["roofline"]["stream_ceiling"] = _ceiling(r["stream"])

    if not args.no_extra:
        extra = []
        for wid in (4,):
            w4 = WORKLOADS[wid]
            r4 = bench_decode(w4, args.extra_steps, 3, 0)
            a4 = r4["step_bytes"] / (r4["kernel_ms"] / 1e3) / 1e9
            d4 = r4["decode_bytes"] / (r4["decode_only_ms"] / 1e3) / 1e9
            extra.append({"workload": w4.name, "value": round(r4["step_bytes"] / (r4["ms_per_step"] / 1e3) / 1e9, 2),
                          "unit": "GB/s", "ms_per_step": round(r4["ms_per_step"], 5),
                          "two_launch_ms_per_step": round(r4["two_launch_ms_per_step"], 5),
                          "eager_ms_per_step": round(r4["eager_ms_per_step"], 5),
                          "roofline": {"bound": "hbm", "kernel": "decode_kernel (gqa_append_decode)",
                                       "achieved": round(a4, 2), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(a4 / PEAK_HBM_GBS, 4),
                                       "kernel_ms": round(r4["kernel_ms"], 5),
                                       "decode_only": {"kernel_ms": round(r4["decode_only_ms"], 5),
                                                       "achieved": round(d4, 2),
                                                       "frac": round(d4 / PEAK_HBM_GBS, 4)}}})
            if r4["stream"] is not None:
                extra[-1]["roofline"]["stream_ceiling"] = _ceiling(r4["stream"])
            del r4
        for wid in (3, 5):
            wp = WORKLOADS[wid]
            rp = bench_prefill(wp, args.extra_steps, 3)
            tf = rp["flops"] / (rp["kernel_ms"] / 1e3) / 1e12
            extra.append({"workload": wp.name,
                          "value": round(rp["flops"] / (rp["ms_per_step"] / 1e3) / 1e12, 2),
                          "unit": "TFLOP/s", "ms_per_step": round(rp["ms_per_step"], 5),
                          "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                       "kernel_ms": round(rp["kernel_ms"], 5), "flops_per_launch": rp["flops"]}})
            torch.cuda.empty_cache()
        extra.append(bench_prefill_d256(args.extra_steps))
        torch.cuda.empty_cache()
        line["extra"] = extra
        line["rotary"] = bench_rotary(args.extra_steps, 3)
        line["rolling"] = bench_rolling(5)
        line["masks"] = bench_masks(3)
        line["fp8"] = bench_fp8(5)

    line["peaks_measured"] = peaks_measured()
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w, r["inputs"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
