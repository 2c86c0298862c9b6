"""INT8 KV cache with per-KV-head scales -- TEST INFRASTRUCTURE ONLY.

The product path never imports this module; it imports nothing but NumPy and
the oracle's own ``materialized`` module.

The pages name quantized KV caches (i8/i4/f8) only as outside their own
scope ([NPUW] "Support GQA sliding-window and smooth-softmax in
DecomposeGQA", section "smooth_softmax / head_sink"; [tract] "onnx: import
GroupQueryAttention decode steps and its internal rotary", section "What
changed": quantized KV rejected).  Every rule below is therefore a reading,
the plainest one that keeps the attention of the other modules unchanged:

* Format: signed 8-bit integer codes, symmetric (zero maps to zero), range
  -127 .. 127 (the code -128 is never written, so the range is symmetric).
* Scales: one fp32 scale per KV head for the K cache and one per KV head for
  the V cache (the same for every batch); the cache holds codes c with
  K[b, g] = c * k_scale[g] (V likewise).
* Quantizing a new row element x (upcast exactly to fp32): t = x * r in fp32,
  r = fp32(1 / scale[g]) (an fp32 division); the code is t rounded to the
  nearest integer, ties to even, clamped to [-127, 127]; NaN gives 0.
* Attention reads K and V through that dequantization and is otherwise the
  attention of ``oracle.materialized``.
"""

from __future__ import annotations

import numpy as np

from .materialized import append_kv as _append_kv, decode as _decode

__all__ = ["INT8_MAX", "quantize", "append", "dequantize", "decode"]

INT8_MAX = 127


def _per_head(scales, x):
    """fp32 scales [Hkv] broadcast over a [B, Hkv, L, D] array."""
    s = np.asarray(scales, dtype=np.float32)
    if s.ndim != 1 or s.shape[0] != np.asarray(x).shape[1]:
        raise ValueError("one scale per KV head")
    return s[None, :, None, None]


def quantize(x, scales):
    """int8 codes of x [B, Hkv, L, D] with per-KV-head scales (see the
    module readings)."""
    x = np.asarray(x, dtype=np.float32)
    r = (np.float32(1.0) / _per_head(scales, x)).astype(np.float32)
    t = (x * r).astype(np.float32)
    t = np.where(np.isnan(t), np.float32(0.0), t)
    q = np.clip(np.rint(t), -INT8_MAX, INT8_MAX)   # rint: nearest integer, ties to even
    return q.astype(np.int8)


def dequantize(codes, scales):
    """float64 values of int8 codes [B, Hkv, L, D] with per-KV-head scales."""
    codes = np.asarray(codes, dtype=np.int8)
    return codes.astype(np.float64) * _per_head(scales, codes).astype(np.float64)


def append(k_codes, v_codes, k_new, v_new, seqlens_k, k_scales, v_scales):
    """Quantize the step's rows and write them into the code caches (slots as
    ``oracle.materialized.append_kv``); returns new int8 arrays."""
    kq = quantize(k_new, k_scales).astype(np.float64)
    vq = quantize(v_new, v_scales).astype(np.float64)
    kc, vc = _append_kv(np.asarray(k_codes, dtype=np.float64), np.asarray(v_codes, dtype=np.float64),
                        kq, vq, seqlens_k)
    return kc.astype(np.int8), vc.astype(np.int8)


def decode(q, k_codes, v_codes, seqlens_k, *, k_scales, v_scales, **kw):
    """Decode against code caches: attention over dequantized K and V."""
    return _decode(q, dequantize(k_codes, k_scales), dequantize(v_codes, v_scales), seqlens_k, **kw)
