"""Seeded synthetic inputs for the five reference workloads and for ad-hoc shapes.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic, so both the HIP path's tests and the oracle's tests can
take their inputs from it.

Recipe (identical for every workload):
  * ``numpy.random.default_rng(seed)``; seed defaults to 1000 + workload id;
  * float32 ``standard_normal`` draws in the fixed order q, k, v (for decode
    the full cache, stale slots included), k_new, v_new, head_sink, then the
    per-batch lengths;
  * q/k/v/k_new/v_new multiplied by ``value_scale`` (0.5 where the workload
    says N(0,1)*0.5), then rounded to the device dtype by torch
    (round-to-nearest-even); head_sink stays float32;
  * layouts: q/out [B, Hq, L, D], k/v [B, Hkv, L or capacity, D], contiguous.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """Shape and attribute set of one synthetic workload.

    kind == "prefill": Lq query rows against Lk keys (empty past).
    kind == "decode": Lq = curr new tokens, Lk = cache capacity.
    seqlens: decode only -- ("uniform", lo, hi) draws seqlens_k from
      integers(lo, hi) (half-open), ("const", n) sets every seqlens_k to n.
    nonpad: prefill only -- per-batch nonpad_kv_seqlen, or None.
    """

    name: str
    kind: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Lq: int
    Lk: int
    window: int = -1
    causal: bool = True
    softcap: float = 0.0
    smooth_softmax: bool = False
    head_sink: bool = False
    value_scale: float = 1.0
    seqlens: Optional[tuple] = None
    nonpad: Optional[tuple] = None
    scale: Optional[float] = None
    seed: int = 0

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny_prefill_fp32", "prefill", "f32", B=1, Hq=4, Hkv=2, D=32,
                Lq=64, Lk=64, window=16, smooth_softmax=True, head_sink=True,
                seed=1001),
    2: Workload("decode_1tok_bf16", "decode", "bf16", B=8, Hq=32, Hkv=8, D=128,
                Lq=1, Lk=4096, window=-1, smooth_softmax=True,
                seqlens=("uniform", 1024, 4096), seed=1002),
    3: Workload("long_prefill_bf16", "prefill", "bf16", B=1, Hq=32, Hkv=8, D=128,
                Lq=8192, Lk=8192, window=4096, value_scale=0.5, seed=1003),
    4: Workload("spec_decode_bf16", "decode", "bf16", B=4, Hq=16, Hkv=8, D=256,
                Lq=4, Lk=32768, window=4096, head_sink=True, softcap=50.0,
                seqlens=("const", 16387), seed=1004),
    5: Workload("gqa_prefill_large_bf16", "prefill", "bf16", B=2, Hq=64, Hkv=8,
                D=128, Lq=32768, Lk=32768, window=8192, head_sink=True,
                value_scale=0.5, nonpad=(32768, 24576), seed=1005),
}


def _draw(rng, shape, value_scale, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if value_scale != 1.0:
        x *= np.float32(value_scale)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype])


def generate(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of ``w`` as CPU torch tensors (see the module recipe).

    prefill -> q, k, v, head_sink, nonpad
    decode  -> q, k_cache, v_cache, k_new, v_new, head_sink, seqlens_k
    Absent optional inputs are None.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = {}
    out["q"] = _draw(rng, (w.B, w.Hq, w.Lq, w.D), w.value_scale, w.dtype)
    kv_shape = (w.B, w.Hkv, w.Lk, w.D)
    if w.kind == "prefill":
        out["k"] = _draw(rng, kv_shape, w.value_scale, w.dtype)
        out["v"] = _draw(rng, kv_shape, w.value_scale, w.dtype)
    elif w.kind == "decode":
        out["k_cache"] = _draw(rng, kv_shape, w.value_scale, w.dtype)
        out["v_cache"] = _draw(rng, kv_shape, w.value_scale, w.dtype)
        new_shape = (w.B, w.Hkv, w.Lq, w.D)
        out["k_new"] = _draw(rng, new_shape, w.value_scale, w.dtype)
        out["v_new"] = _draw(rng, new_shape, w.value_scale, w.dtype)
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    out["head_sink"] = (torch.from_numpy(rng.standard_normal(w.Hq, dtype=np.float32))
                        if w.head_sink else None)
    if w.kind == "decode":
        if w.seqlens is None:
            raise ValueError("decode workload needs seqlens")
        if w.seqlens[0] == "uniform":
            s = rng.integers(w.seqlens[1], w.seqlens[2], size=w.B)
        elif w.seqlens[0] == "const":
            s = np.full(w.B, w.seqlens[1])
        elif w.seqlens[0] == "list":
            s = np.asarray(w.seqlens[1])
        else:
            raise ValueError(f"unknown seqlens recipe {w.seqlens!r}")
        out["seqlens_k"] = torch.from_numpy(s.astype(np.int32))
    else:
        out["nonpad"] = (torch.tensor(w.nonpad, dtype=torch.int64)
                         if w.nonpad is not None else None)
    return out


def rotary_tables(max_pos: int, D: int, base: float = 10000.0):
    """cos and sin tables [max_pos, D/2] (float32 CPU tensors) of the usual
    rotary frequencies: row p, column i holds the angle p * base^(-2i/D).
    These are inputs a caller supplies (a model's position tables), not part
    of the attention arithmetic."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


def to_f64(t):
    """Exact upcast of a (CPU or device) tensor to a float64 NumPy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def staircase(n: int, step: float, period: int) -> np.ndarray:
    """Logit levels of a staircase over key positions 0..n-1: position j sits
    on level floor(j / period), at height step * level (nats)."""
    return step * (np.arange(n) // period).astype(np.float64)


def bursts(n: int, height: float, period: int, width: int, offset: int = 0) -> np.ndarray:
    """Logit levels that are 0 except for bursts of `width` positions at
    `height` (nats) ending every `period` positions (shifted by `offset`)."""
    j = np.arange(n) + offset
    return np.where(j % period >= period - width, height, 0.0)


def shape_logits(w: Workload, d: dict, levels: np.ndarray, seed: int, *, a: float = 1.0,
                 q_noise: float = 0.1, k_noise: float = 0.3, v_level: float = 0.7,
                 v_noise: float = 0.5, flip: Optional[np.ndarray] = None) -> dict:
    """Inputs whose scaled logits follow a prescribed profile over key positions.

    Every query row is a * u plus noise and key position j is
    levels[j] / (a * |u|^2 * scale) * u plus noise, for one fixed +-1 vector u,
    so that the scaled logit of any query against position j is about
    levels[j] nats (plus noise of a few tenths).  Values are +-v_level plus
    noise, the sign given by `flip` (default: alternating with the level's
    rank), so that the result depends on how the softmax weighs different
    levels.  Decode inputs place new token t of batch b at position
    seqlens_k[b] + 1 - curr + t.  The rest of `d` (lengths, sinks) is kept.
    This designs inputs; it computes no attention."""
    rng = np.random.default_rng(seed)
    D, scale = w.D, w.sm_scale
    u = rng.choice([-1.0, 1.0], size=D)
    b_of = levels / (a * D * scale)                       # u-coefficient of each position
    if flip is None:
        _, rank = np.unique(levels, return_inverse=True)
        flip = np.where(rank % 2 == 0, 1.0, -1.0)
    dt = TORCH_DTYPES[w.dtype]

    def rows(shape, coef, noise, sign=None):
        if sign is not None:
            x = sign[..., None] * v_level + noise * rng.standard_normal(shape + (D,))
        else:
            x = coef[..., None] * u + noise * rng.standard_normal(shape + (D,))
        return torch.from_numpy(x.astype(np.float32)).to(dt)

    out = dict(d)
    out["q"] = rows((w.B, w.Hq, w.Lq), np.full((w.B, w.Hq, w.Lq), a), q_noise)
    kv = (w.B, w.Hkv, w.Lk)
    pos = np.broadcast_to(np.arange(w.Lk), kv)
    k_name, v_name = ("k", "v") if w.kind == "prefill" else ("k_cache", "v_cache")
    out[k_name] = rows(kv, b_of[pos], k_noise)
    out[v_name] = rows(kv, None, v_noise, sign=flip[pos])
    if w.kind == "decode":
        s = d["seqlens_k"].numpy().astype(np.int64)
        npos = (s + 1 - w.Lq)[:, None, None] + np.arange(w.Lq)[None, None, :]
        npos = np.broadcast_to(np.clip(npos, 0, w.Lk - 1), (w.B, w.Hkv, w.Lq))
        out["k_new"] = rows((w.B, w.Hkv, w.Lq), b_of[npos], k_noise)
        out["v_new"] = rows((w.B, w.Hkv, w.Lq), None, v_noise, sign=flip[npos])
    return out
