"""Algorithmic work of one call, from the closed-form allowed interval.

For a query at absolute position p the allowed keys form one interval
[lo, hi] (each constraint of the causal band, the window and the valid length
is a half-line in the key index):
    hi = min(p, valid - 1)        (causal; valid - 1 without the causal band)
    lo = max(0, p - W + 1)        (0 with the window off)
This follows the window rule of "[NPUW] Support GQA sliding-window and
smooth-softmax in DecomposeGQA" (section "Sliding window (local_window_size)")
and the lower-bound-on-the-band description of "Add sliding windows to the
off-graph KV-cache reference" (section "Summary").

Counts used by the benchmark's roofline figures:
  * FLOPs = 4 * D per kept (query, key) pair: QK^T and PV, each 2*D, on the
    kept band only (softmax work and masked pairs are not counted);
  * decode bytes = the K and V rows of the union of the kept intervals, read
    once per (batch, KV head), plus Q in and O out.  Stale slots, keys outside
    the window and the G-fold re-use of K/V by query heads are not counted.
"""

from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}


def intervals(q_abs, valid, causal: bool, window: int):
    """(lo, hi, n) arrays for absolute query positions ``q_abs``."""
    q_abs = np.asarray(q_abs, dtype=np.int64)
    hi = np.minimum(q_abs, valid - 1) if causal else np.full_like(q_abs, valid - 1)
    lo = np.maximum(0, q_abs - window + 1) if window != -1 else np.zeros_like(q_abs)
    n = np.maximum(0, hi - lo + 1)
    return lo, hi, n


def prefill_pairs_per_batch(B, Lq, Lk, causal, window, nonpad=None):
    """Kept pairs per query head, one entry per batch."""
    valid = np.full(B, Lk) if nonpad is None else np.asarray(nonpad).reshape(B)
    q_abs = (Lk - Lq) + np.arange(Lq)
    return np.array([int(intervals(q_abs, int(valid[b]), causal, window)[2].sum())
                     for b in range(B)], dtype=np.int64)


def prefill_flops(B, Hq, D, Lq, Lk, causal, window, nonpad=None) -> int:
    return 4 * D * Hq * int(prefill_pairs_per_batch(B, Lq, Lk, causal, window, nonpad).sum())


def decode_pairs(seqlens_k, curr, causal, window) -> int:
    """Kept pairs per query head, summed over the batch."""
    total = np.asarray(seqlens_k, dtype=np.int64).reshape(-1) + 1
    n = 0
    for t in total:
        q_abs = (t - curr) + np.arange(curr)
        n += int(intervals(q_abs, int(t), causal, window)[2].sum())
    return n


def decode_union_keys(seqlens_k, curr, causal, window):
    """Length of the union of kept intervals per batch (all KV heads alike)."""
    total = np.asarray(seqlens_k, dtype=np.int64).reshape(-1) + 1
    out = []
    for t in total:
        q_abs = (t - curr) + np.arange(curr)
        lo, hi, n = intervals(q_abs, int(t), causal, window)
        keep = n > 0
        out.append(int(hi[keep].max() - lo[keep].min() + 1) if keep.any() else 0)
    return np.array(out, dtype=np.int64)


def decode_bytes(seqlens_k, curr, Hq, Hkv, D, dtype, causal, window, kv_dtype=None) -> int:
    """``kv_dtype`` ("fp8" for an FP8 cache) sizes the K/V rows when it
    differs from the type of Q and O."""
    e = ELEM_BYTES[dtype]
    keys = int(decode_union_keys(seqlens_k, curr, causal, window).sum())
    B = len(np.asarray(seqlens_k).reshape(-1))
    kv = 2 * keys * Hkv * D * ELEM_BYTES[kv_dtype or dtype]
    qo = 2 * B * Hq * curr * D * e
    return kv + qo


def decode_flops(seqlens_k, curr, Hq, D, causal, window) -> int:
    return 4 * D * Hq * decode_pairs(seqlens_k, curr, causal, window)


def append_bytes(B, Hkv, curr, D, dtype) -> int:
    """K and V rows read from the step buffers and written into the cache."""
    return 2 * 2 * B * Hkv * curr * D * ELEM_BYTES[dtype]


def rotary_bytes(rows: int, D: int, dtype: str, positions: int) -> int:
    """Rotary embedding of `rows` rows of D elements at `positions` distinct
    positions: every row read and written once, and the cos and sin table
    rows (D/2 fp32 each) of those positions read once."""
    return 2 * rows * D * ELEM_BYTES[dtype] + positions * D * 4


def append_rotary_bytes(B, Hq, Hkv, curr, D, dtype) -> int:
    """One decode step's append with rotary: the new K and V rows read and
    written into the cache, the query rows read and written turned, and the
    table rows of the B * curr positions read."""
    e = ELEM_BYTES[dtype]
    return 2 * (2 * B * Hkv + B * Hq) * curr * D * e + B * curr * D * 4

