"""FP8 (E4M3) KV cache -- TEST INFRASTRUCTURE ONLY.

The product path never imports this module; it imports nothing but NumPy and
the oracle's own ``materialized`` module.

The pages name quantized KV caches (i8/i4/f8) only as outside their own
scope ([NPUW] "Support GQA sliding-window and smooth-softmax in
DecomposeGQA", section "smooth_softmax / head_sink"; [tract] "onnx: import
GroupQueryAttention decode steps and its internal rotary", section "What
changed": quantized KV rejected).  Everything below is therefore a reading,
the plainest one that keeps the attention of the other modules unchanged:

* Format: the OCP 8-bit floating-point E4M3 encoding -- 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits.  Exponent field E in 1..15
  gives (-1)^s 2^(E-7) (1 + M/8); E = 0 gives the subnormals (-1)^s 2^-6 M/8;
  the two codes S.1111.111 are NaN; there are no infinities; the largest
  finite magnitude is 448.
* Scales: one fp32 scale for the K cache and one for the V cache; the cache
  holds codes c with K = decode(c) * k_scale (V likewise).
* Quantizing a new row element x (upcast exactly to fp32): t = x * r in fp32,
  r = fp32(1 / scale) (an fp32 division); the code of the E4M3 value nearest
  to t, ties to the even code; magnitudes beyond 448 saturate to 448, so the
  cache stays finite; a negative t that rounds to zero keeps its sign.
* Attention reads K and V through that dequantization and is otherwise the
  attention of ``oracle.materialized``.
"""

from __future__ import annotations

import numpy as np

from .materialized import append_kv as _append_kv, decode as _decode

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize", "append", "dequantize", "decode"]

E4M3_MAX = 448.0


def _value_of_code(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * 2.0 ** -6 * (m / 8.0)
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


_TABLE = np.array([_value_of_code(c) for c in range(256)], dtype=np.float64)
# the finite non-negative values, in code order (which is value order)
_POS = _TABLE[:0x7F]


def e4m3_decode(codes):
    """float64 values of uint8 E4M3 codes (NaN for the two NaN codes)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(t):
    """uint8 codes of the E4M3 values nearest to ``t`` (ties to the even
    code), magnitudes beyond 448 saturated to 448, NaN to 0x7F."""
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(t), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(t), np.uint8(0x7F), code).astype(np.uint8)


def quantize(x, scale: float):
    """Codes of x / scale as the cache stores them (see the module readings)."""
    r = np.float32(1.0) / np.float32(scale)
    t = np.asarray(x, dtype=np.float32) * r
    return e4m3_encode(t.astype(np.float64))


def append(k_codes, v_codes, k_new, v_new, seqlens_k, k_scale: float, v_scale: float):
    """Quantize the step's rows and write them into the code caches (slots as
    ``oracle.materialized.append_kv``); returns new uint8 arrays."""
    kq = quantize(k_new, k_scale).astype(np.float64)
    vq = quantize(v_new, v_scale).astype(np.float64)
    kc, vc = _append_kv(np.asarray(k_codes, dtype=np.float64), np.asarray(v_codes, dtype=np.float64),
                        kq, vq, seqlens_k)
    return kc.astype(np.uint8), vc.astype(np.uint8)


def dequantize(codes, scale: float):
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def decode(q, k_codes, v_codes, seqlens_k, *, k_scale: float, v_scale: float, **kw):
    """Decode against code caches: attention over dequantized K and V."""
    return _decode(q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), seqlens_k, **kw)
