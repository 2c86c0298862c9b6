"""Rotary position embedding for the oracle -- TEST INFRASTRUCTURE ONLY.

The product path never imports this module; it imports nothing but NumPy and
the oracle's own ``materialized`` module.

Source: [tract] "onnx: import GroupQueryAttention decode steps and its
internal rotary" (tract pull request), section "What changed", the do_rotary
item:

* the node rotates Q and K itself, from a cos table and a sin table whose
  halves are widened to the head size;
* a first prompt takes positions 0 .. S-1, a generated token takes position
  seqlens_k;
* K is rotated before it is written into the cache, so the cache holds
  rotated keys.

Readings taken where the page leaves a step open
------------------------------------------------
* Pairing: each table has D/2 columns and is widened by using it for both
  halves, so element i pairs with element i + D/2 (i < D/2).  The pair turns
  by the angle whose cosine and sine are cos[p, i] and sin[p, i]:
  (a, b) -> (a c - b s, b c + a s).  This is the turn of the complex number
  a + i b by e^{i theta}, the rotate-half form.  The interleaved form
  (pairing 2i with 2i + 1) is not covered.
* Tables: the caller supplies both, float, shape [max_pos, D/2], row p for
  position p.
* Positions are absolute and equal the cache slot: prefill query row i sits
  at q_offset + i (0 .. S-1 for a first prompt, where Lq = Lk) and key j at
  j; new decode token t sits at total_b - curr + t with total_b =
  seqlens_k[b] + 1 (seqlens_k[b] itself for a single generated token).
* A position outside [0, max_pos) is an error.
"""

from __future__ import annotations

import numpy as np

from .materialized import append_kv

__all__ = ["rotate", "prefill_positions", "decode_positions", "rotate_prefill", "append_kv_rotary"]


def rotate(x, positions, cos_table, sin_table):
    """Turn each (x_i, x_{i+D/2}) pair of the rows of ``x`` by its row's angle.

    x: [..., D] (D even); positions: integers broadcastable to x.shape[:-1];
    cos_table, sin_table: [max_pos, D/2].  Returns float64 of x's shape.
    """
    x = np.asarray(x, dtype=np.float64)
    cos_table = np.asarray(cos_table, dtype=np.float64)
    sin_table = np.asarray(sin_table, dtype=np.float64)
    D = x.shape[-1]
    if D % 2 != 0:
        raise ValueError("rotary needs an even head size")
    half = D // 2
    if cos_table.shape != sin_table.shape or cos_table.ndim != 2 or cos_table.shape[1] != half:
        raise ValueError("cos/sin tables must both be [max_pos, D/2]")
    p = np.broadcast_to(np.asarray(positions, dtype=np.int64), x.shape[:-1])
    if p.size and (p.min() < 0 or p.max() >= cos_table.shape[0]):
        raise ValueError("rotary position outside the tables")
    c = cos_table[p]
    s = sin_table[p]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def prefill_positions(Lq: int, Lk: int):
    """(query positions, key positions) of a prompt on an empty past."""
    return (Lk - Lq) + np.arange(Lq), np.arange(Lk)


def decode_positions(seqlens_k, curr: int):
    """[B, curr] positions of the new tokens: total_b - curr + t."""
    total = np.asarray(seqlens_k, dtype=np.int64).reshape(-1) + 1
    return total[:, None] - curr + np.arange(curr)[None, :]


def rotate_prefill(q, k, cos_table, sin_table):
    """Rotated (q, k) of a prompt: q [B, Hq, Lq, D], k [B, Hkv, Lk, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    pq, pk = prefill_positions(q.shape[2], k.shape[2])
    return rotate(q, pq, cos_table, sin_table), rotate(k, pk, cos_table, sin_table)


def append_kv_rotary(k_cache, v_cache, q, k_new, v_new, seqlens_k, cos_table, sin_table):
    """One decode step's inputs with rotary: (q_rot, k_cache', v_cache').

    The curr new K rows are turned at their positions and then concatenated
    onto the past (V unchanged); the curr query rows are turned at the same
    positions.  Inputs are left untouched.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    curr = k_new.shape[2]
    if q.shape[2] != curr:
        raise ValueError("q and k_new must hold the same new tokens")
    pos = decode_positions(seqlens_k, curr)[:, None, :]  # [B, 1, curr] over heads
    k_rot = rotate(k_new, pos, cos_table, sin_table)
    q_rot = rotate(q, pos, cos_table, sin_table)
    kc, vc = append_kv(k_cache, v_cache, k_rot, v_new, seqlens_k)
    return q_rot, kc, vc
