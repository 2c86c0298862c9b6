"""Materialized float64 oracle for windowed grouped-query attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module, and this module imports nothing but NumPy.

What it computes, and where each piece comes from
-------------------------------------------------
Sources are the four pages this project is built from, cited by title and
section:

* [NPUW] "Support GQA sliding-window and smooth-softmax in DecomposeGQA"
  (OpenVINO pull request), sections "Sliding window (local_window_size)" and
  "smooth_softmax / head_sink".
* [tract] "onnx: import GroupQueryAttention decode steps and its internal
  rotary" (tract pull request), sections "What changed" and "On the mask
  sentinel".
* [executorch] "Add sliding windows to the off-graph KV-cache reference"
  (executorch pull request), section "Summary".
* [ALC] "Attention Kernel Design" (onnx-light-cpu docs), sections "Layouts and
  semantics", "Compute paths" and "Scheduling, precision, and invariants".

The structure is the materialized path of [ALC] "Compute paths": form every
score of a block of query rows against every key, mask, softmax, multiply by
V.  Everything is float64; inputs are whatever the caller passes (the tests
pass values already rounded to the device dtype, upcast exactly).

For batch b, query head h, query row i and key slot j:

1. Head map: K/V head g = h // G with G = Hq / Hkv, no K/V copies
   ([ALC] "Layouts and semantics").
2. Absolute positions: query row i sits at q_abs = q_offset[b] + i and key
   slot j at position j.  Prefill uses q_offset = Lk - Lq, the bottom-right
   band ([tract] "What changed": the band built from Range(kv_len - q_len,
   kv_len)); decode uses q_offset = total_b - curr, total_b = seqlens_k[b] + 1
   ([NPUW] "Sliding window": q_abs(i) = (total - curr) + i).
3. Allowed set, evaluated elementwise: j < valid_b, and j <= q_abs when
   causal, and q_abs - j < W when the window is on ([NPUW] "Sliding window":
   keys with q_abs - k_abs >= local_window_size are masked; [executorch]
   "Summary": the window is a lower bound added to the causal band).
4. Logit x = scale * <q_i, k_j>; with softcap c > 0, x <- c * tanh(x / c)
   ([ALC] "Layouts and semantics" lists softcap).
5. Softmax over the allowed keys, with an optional extra logit s_h that
   enters the denominator only ([NPUW] "smooth_softmax / head_sink": the sink
   joins the softmax and is sliced out; head_sink per head, or 0 for plain
   smooth_softmax).
6. A row with no allowed key gives exactly 0 ([ALC] "Scheduling, precision,
   and invariants").  Masking is a select, never indicator * sentinel
   ([tract] "On the mask sentinel").
7. An optional caller mask broadcast over [B, Hq, Lq, Lk] ([ALC] "Layouts
   and semantics": boolean and float additive broadcast masks): a boolean
   mask takes the keys where it is False out of the allowed set; an additive
   mask adds its value to the scaled logit ([tract] "What changed":
   attention_bias summed with the band).

Readings taken where the pages leave a step open
------------------------------------------------
* head order g = h // G (blocked, the repeat_interleave order);
* W counts keys including the query's own position; W = 1 is self-only;
  W = -1 switches the window off; any other W < 1 is invalid;
* softcap acts on the scaled logit, before masking; the sink logit is neither
  scaled nor capped;
* a head_sink array turns the sink on whether or not smooth_softmax is set;
  smooth_softmax alone means s_h = 0;
* causal = False is defined only with the window off (the window is one-sided);
* nonpad_kv_seqlen masks keys j >= nonpad_b but does not move q_offset;
* key slots that no query row of a (batch, head, row-block) may see never
  influence the result, whatever they hold (stale cache slots, padding); a
  slot that some row may see must hold finite values;
* a boolean mask is True where the query may attend; an additive mask is
  added to the scaled logit before softcap (scale, bias, cap), a key whose
  added value is -inf leaves the allowed set (so a row whose every key has
  -inf is 0), and the sink logit gets no bias.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "allowed",
    "softcap_fn",
    "sink_logits",
    "attention",
    "prefill",
    "decode",
    "append_kv",
]


def allowed(q_abs, j, valid, causal: bool, window: int):
    """Elementwise allowed-set predicate (step 3 of the module docstring).

    ``q_abs`` and ``j`` broadcast against each other; ``valid`` is a scalar.
    """
    q_abs, j = np.broadcast_arrays(np.asarray(q_abs), np.asarray(j))
    ok = (j >= 0) & (j < valid)
    if causal:
        ok = ok & (j <= q_abs)
    if window != -1:
        ok = ok & ((q_abs - j) < window)
    return ok


def softcap_fn(x, cap: float):
    """c * tanh(x / c) for c > 0, identity for c == 0 (step 4)."""
    if cap > 0:
        return cap * np.tanh(x / cap)
    return x


def sink_logits(num_heads: int, smooth_softmax: bool, head_sink=None):
    """Per-head extra logit s_h, or None when no sink is in play (step 5)."""
    if head_sink is not None:
        s = np.asarray(head_sink, dtype=np.float64).reshape(-1)
        if s.shape[0] != num_heads:
            raise ValueError("head_sink must have one entry per query head")
        return s
    if smooth_softmax:
        return np.zeros(num_heads, dtype=np.float64)
    return None


def _check_attrs(Hq, Hkv, causal, window, softcap, scale):
    if Hq <= 0 or Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("need Hq > 0, Hkv > 0 and Hq % Hkv == 0")
    if window != -1 and window < 1:
        raise ValueError("local_window_size must be -1 or >= 1")
    if not causal and window != -1:
        raise ValueError("a window needs the causal band")
    if softcap < 0:
        raise ValueError("softcap must be >= 0")
    if not scale > 0:
        raise ValueError("scale must be > 0")


def attention(q, k, v, q_offset, valid, *, scale: float, causal: bool = True,
              window: int = -1, softcap: float = 0.0, sink=None, rows=None,
              mask=None, chunk: int = 256):
    """Materialized attention over arbitrary per-batch offsets.

    q: [B, Hq, Lq, D]; k, v: [B, Hkv, Lk, D]; q_offset, valid: length-B ints.
    ``sink`` is None or a length-Hq array of natural-log logits.  ``rows``
    optionally restricts the computation to those query rows (each row is
    independent, so a subset is the same arithmetic); the result then has
    len(rows) rows.  ``mask`` is None or an array broadcastable to
    [B, Hq, Lq, Lk]: boolean (True = may attend) or float (added to the
    scaled logit).  Returns float64 [B, Hq, len(rows), D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError("q/k/v shapes disagree")
    _check_attrs(Hq, Hkv, causal, window, softcap, scale)
    G = Hq // Hkv
    q_offset = np.broadcast_to(np.asarray(q_offset, dtype=np.int64), (B,))
    valid = np.broadcast_to(np.asarray(valid, dtype=np.int64), (B,))
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    if mask is not None:
        mask = np.asarray(mask)
        if mask.dtype != np.bool_:
            mask = mask.astype(np.float64)
        mask = np.broadcast_to(mask, (B, Hq, Lq, Lk))
    out = np.zeros((B, Hq, rows.shape[0], D), dtype=np.float64)
    j = np.arange(Lk)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        for b in range(B):
            for h in range(Hq):
                g = h // G
                kbg = k[b, g]
                vbg = v[b, g]
                s = None if sink is None else float(sink[h])
                for c0 in range(0, rows.shape[0], chunk):
                    r = rows[c0:c0 + chunk]
                    q_abs = q_offset[b] + r
                    M = allowed(q_abs[:, None], j[None, :], valid[b], causal, window)
                    X = scale * (q[b, h, r] @ kbg.T)
                    if mask is not None and mask.dtype == np.bool_:
                        M = M & mask[b, h, r]
                    elif mask is not None:
                        M = M & (mask[b, h, r] > -np.inf)
                        X = X + np.where(M, mask[b, h, r], 0.0)
                    X = softcap_fn(X, softcap)
                    X = np.where(M, X, -np.inf)
                    m = X.max(axis=1)
                    if s is not None:
                        m = np.maximum(m, s)
                    m = np.where(np.isfinite(m), m, 0.0)
                    E = np.where(M, np.exp(X - m[:, None]), 0.0)
                    Z = E.sum(axis=1)
                    if s is not None:
                        Z = Z + np.exp(s - m)
                    # slots no row of this block may see are excluded outright
                    seen = M.any(axis=0)
                    vis = np.where(seen[:, None], vbg, 0.0)
                    O = (E @ vis) / Z[:, None]
                    O[~M.any(axis=1)] = 0.0
                    out[b, h, c0:c0 + r.shape[0]] = O
    return out


def prefill(q, k, v, *, scale: float, causal: bool = True, window: int = -1,
            softcap: float = 0.0, smooth_softmax: bool = False, head_sink=None,
            nonpad_kv_seqlen=None, rows=None, mask=None):
    """Prompt attention on an empty past: q_offset = Lk - Lq for every batch.

    ``nonpad_kv_seqlen`` (length B, 0 <= n <= Lk) masks keys j >= n without
    moving the causal offset.
    """
    q = np.asarray(q)
    B, Hq, Lq, _ = q.shape
    Lk = np.asarray(k).shape[2]
    if nonpad_kv_seqlen is None:
        valid = np.full(B, Lk, dtype=np.int64)
    else:
        valid = np.asarray(nonpad_kv_seqlen, dtype=np.int64).reshape(B)
        if (valid < 0).any() or (valid > Lk).any():
            raise ValueError("nonpad_kv_seqlen must lie in [0, Lk]")
    q_offset = np.full(B, Lk - Lq, dtype=np.int64)
    sink = sink_logits(Hq, smooth_softmax, head_sink)
    return attention(q, k, v, q_offset, valid, scale=scale, causal=causal,
                     window=window, softcap=softcap, sink=sink, rows=rows, mask=mask)


def decode(q, k_cache, v_cache, seqlens_k, *, scale: float, causal: bool = True,
           window: int = -1, softcap: float = 0.0, smooth_softmax: bool = False,
           head_sink=None, rows=None, mask=None):
    """Decode of curr = q.shape[2] new tokens against a cache already holding them.

    seqlens_k[b] = total_b - 1: the newest token sits at slot seqlens_k[b];
    the curr query rows are at positions total_b - curr ... total_b - 1 and
    the cache holds valid keys in slots [0, total_b).
    """
    q = np.asarray(q)
    B, Hq, curr, _ = q.shape
    cap = np.asarray(k_cache).shape[2]
    total = np.asarray(seqlens_k, dtype=np.int64).reshape(B) + 1
    if (total < curr).any() or (total > cap).any():
        raise ValueError("need curr <= seqlens_k + 1 <= capacity")
    sink = sink_logits(Hq, smooth_softmax, head_sink)
    return attention(q, k_cache, v_cache, total - curr, total, scale=scale,
                     causal=causal, window=window, softcap=softcap, sink=sink,
                     rows=rows, mask=mask)


def append_kv(k_cache, v_cache, k_new, v_new, seqlens_k):
    """Concatenate curr new K/V rows onto the past: slots total_b - curr ...
    total_b - 1 ([tract] "What changed": present = concat(past, step)).

    Returns new arrays; the inputs are left untouched.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, _, curr, _ = np.asarray(k_new).shape
    cap = kc.shape[2]
    total = np.asarray(seqlens_k, dtype=np.int64).reshape(B) + 1
    for b in range(B):
        t = int(total[b])
        if t < curr or t > cap:
            raise ValueError("need curr <= seqlens_k + 1 <= capacity")
        kc[b, :, t - curr:t] = k_new[b]
        vc[b, :, t - curr:t] = v_new[b]
    return kc, vc
