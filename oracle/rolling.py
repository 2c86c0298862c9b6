"""Rolling (ring-buffer) KV cache of a windowed layer -- TEST INFRASTRUCTURE ONLY.

The product path never imports this module; it imports nothing but NumPy and
the oracle's own ``materialized`` module.

Sources:

* [NPUW] "Support GQA sliding-window and smooth-softmax in DecomposeGQA",
  section "Sliding window (local_window_size)": sliding_window_cache names
  the physical rolling KV buffer, and applying the window as a mask over the
  full cache gives the same attention result as that buffer.
* [executorch] "Add sliding windows to the off-graph KV-cache reference",
  section "Summary": the reference masks and does not evict.

Readings taken where the pages leave a step open
------------------------------------------------
* A rolling cache of C slots per (batch, KV head) keeps the token at
  absolute position p in slot p mod C; appending a step writes its curr rows
  to the slots of positions total_b - curr .. total_b - 1 (total_b =
  seqlens_k[b] + 1), overwriting the oldest tokens.  Positions are no longer
  bounded by C.
* Decode is the windowed attention of the full history, unchanged: the ring
  is only where the keys live.  This holds exactly when every key a step's
  rows may see is still in the ring, i.e. C >= W + curr - 1 (the earliest
  row of the step, at total - curr, reaches back to total - curr - W + 1).
  A rolling cache therefore needs the window on (W >= 1) and that capacity;
  anything else is an error.
"""

from __future__ import annotations

import numpy as np

from .materialized import decode as _decode

__all__ = ["slot_of", "append", "linear_history", "decode"]


def slot_of(p, capacity: int):
    """Ring slot of absolute position p."""
    return np.asarray(p) % capacity


def _totals(seqlens_k, B):
    return np.asarray(seqlens_k, dtype=np.int64).reshape(B) + 1


def append(k_ring, v_ring, k_new, v_new, seqlens_k):
    """Write the step's rows into their ring slots; returns new arrays."""
    kr = np.array(k_ring, copy=True)
    vr = np.array(v_ring, copy=True)
    B, _, curr, _ = np.asarray(k_new).shape
    C = kr.shape[2]
    if curr > C:
        raise ValueError("a step longer than the ring")
    total = _totals(seqlens_k, B)
    for b in range(B):
        if total[b] < curr:
            raise ValueError("need seqlens_k + 1 >= curr")
        for t in range(curr):
            s = int(slot_of(total[b] - curr + t, C))
            kr[b, :, s] = k_new[b, :, t]
            vr[b, :, s] = v_new[b, :, t]
    return kr, vr


def linear_history(ring, seqlens_k, start: int = 0):
    """[B, H, max_total - start, D] with the key of position j at index
    j - start for the positions the ring still holds (j >= total_b - C);
    older positions, whose slots were overwritten, are NaN (they must never
    be read)."""
    ring = np.asarray(ring, dtype=np.float64)
    B, H, C, D = ring.shape
    total = _totals(seqlens_k, B)
    out = np.full((B, H, int(total.max()) - start, D), np.nan)
    for b in range(B):
        for j in range(max(start, int(total[b]) - C), int(total[b])):
            out[b, :, j - start] = ring[b, :, int(slot_of(j, C))]
    return out


def decode(q, k_ring, v_ring, seqlens_k, *, scale: float, window: int, causal: bool = True,
           softcap: float = 0.0, smooth_softmax: bool = False, head_sink=None):
    """Decode of the curr new tokens (already appended) against a ring."""
    q = np.asarray(q)
    curr = q.shape[2]
    C = np.asarray(k_ring).shape[2]
    if window < 1:
        raise ValueError("a rolling cache needs the window on")
    if C < window + curr - 1:
        raise ValueError("ring too small: need capacity >= window + curr - 1")
    # Only positions from `start` on can be seen by any batch (each batch's
    # rows reach back at most C positions).  The allowed set depends on
    # position differences and on j < total only, so moving every position
    # down by `start` changes nothing; it keeps the materialized history small
    # when positions are large.
    total = _totals(seqlens_k, q.shape[0])
    start = int(max(0, total.min() - C))
    kl = linear_history(k_ring, seqlens_k, start)
    vl = linear_history(v_ring, seqlens_k, start)
    return _decode(q, kl, vl, total - 1 - start, scale=scale, causal=causal, window=window,
                   softcap=softcap, smooth_softmax=smooth_softmax, head_sink=head_sink)
