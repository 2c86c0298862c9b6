"""ctypes binding of libgqa_mi355x (declarations: include/gqa.h).

Argument marshalling only: torch tensors are turned into pointers, element
strides and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  torch is used for device memory (outputs, workspace)
and streams.  If the library is missing, ``load()`` raises -- there is no
fallback path.

The C entry points are exposed under their own names (``gqa_plan``,
``gqa_prefill``, ...) taking ctypes structures; ``Plan`` wraps them for torch
tensors.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_mi355x.so")

GQA_OK = 0
GQA_ERR_INVALID_ARG = 1
GQA_ERR_UNSUPPORTED = 2
GQA_ERR_CAPACITY = 3
GQA_ERR_HIP = 4
STATUS_NAMES = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED",
                3: "GQA_ERR_CAPACITY", 4: "GQA_ERR_HIP"}

GQA_F32, GQA_F16, GQA_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": GQA_F32, "f16": GQA_F16, "bf16": GQA_BF16}

EXPORTED = ("gqa_plan", "gqa_plan_destroy", "gqa_workspace_size", "gqa_prefill",
            "gqa_append_kv", "gqa_decode", "gqa_apply_rotary", "gqa_append_kv_rotary",
            "gqa_prefill_masked", "gqa_decode_masked", "gqa_append_kv_fp8", "gqa_decode_fp8",
            "gqa_decode_fp8_masked", "gqa_decode_noalloc", "gqa_append_decode", "gqa_prefill_rotary",
            "gqa_last_path", "gqa_last_error", "gqa_probe_mfma_peak", "gqa_probe_kv_stream",
            "gqa_append_kv_int8", "gqa_decode_int8", "gqa_decode_int8_masked")
GQA_MASK_BOOL, GQA_MASK_ADDITIVE = 1, 2


class gqa_attrs(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("kv_num_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("local_window_size", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("smooth_softmax", ctypes.c_int32),
        ("use_head_sink", ctypes.c_int32),
        ("is_causal", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("rolling_cache", ctypes.c_int32),
    ]


class gqa_tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_s", ctypes.c_int64),
    ]


class gqa_rotary_tables(ctypes.Structure):
    _fields_ = [
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("max_pos", ctypes.c_int64),
    ]


class gqa_mask(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_q", ctypes.c_int64),
        ("kind", ctypes.c_int),
    ]


gqa_plan_t = ctypes.c_void_p
_lib = None


def load():
    """Load libgqa_mi355x.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m windowed_gqa_kv_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    T, P, I32, I64, S = gqa_tensor, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gqa_plan.argtypes = [ctypes.POINTER(gqa_attrs), I32, I32, I64, ctypes.POINTER(gqa_plan_t)]
    lib.gqa_plan.restype = ctypes.c_int
    lib.gqa_plan_destroy.argtypes = [gqa_plan_t]
    lib.gqa_plan_destroy.restype = None
    lib.gqa_workspace_size.argtypes = [gqa_plan_t]
    lib.gqa_workspace_size.restype = S
    lib.gqa_prefill.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P, S, P]
    lib.gqa_prefill.restype = ctypes.c_int
    lib.gqa_append_kv.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P]
    lib.gqa_append_kv.restype = ctypes.c_int
    lib.gqa_decode.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P, S, P]
    lib.gqa_decode.restype = ctypes.c_int
    RT = ctypes.POINTER(gqa_rotary_tables)
    lib.gqa_apply_rotary.argtypes = [gqa_plan_t, I32, I32, I32, I64, T, T, RT, P]
    lib.gqa_apply_rotary.restype = ctypes.c_int
    lib.gqa_append_kv_rotary.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, T, T, P, RT, P]
    lib.gqa_append_kv_rotary.restype = ctypes.c_int
    MK = ctypes.POINTER(gqa_mask)
    lib.gqa_prefill_masked.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, MK, P]
    lib.gqa_prefill_masked.restype = ctypes.c_int
    lib.gqa_decode_masked.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, MK, P, S, P]
    lib.gqa_decode_masked.restype = ctypes.c_int
    F = ctypes.c_float
    lib.gqa_append_kv_fp8.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, F, F, P]
    lib.gqa_append_kv_fp8.restype = ctypes.c_int
    lib.gqa_decode_fp8.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, F, F, P, S, P]
    lib.gqa_decode_fp8.restype = ctypes.c_int
    lib.gqa_decode_fp8_masked.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, F, F, MK, P, S, P]
    lib.gqa_decode_fp8_masked.restype = ctypes.c_int
    lib.gqa_decode_noalloc.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P]
    lib.gqa_decode_noalloc.restype = ctypes.c_int
    lib.gqa_append_decode.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, T, T, P, P, P, S, P]
    lib.gqa_append_decode.restype = ctypes.c_int
    lib.gqa_prefill_rotary.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, RT, P]
    lib.gqa_prefill_rotary.restype = ctypes.c_int
    lib.gqa_append_kv_int8.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P, P]
    lib.gqa_append_kv_int8.restype = ctypes.c_int
    lib.gqa_decode_int8.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P, P, P, S, P]
    lib.gqa_decode_int8.restype = ctypes.c_int
    lib.gqa_decode_int8_masked.argtypes = [gqa_plan_t, I32, I32, I64, T, T, T, T, P, P, P, P, MK, P, S, P]
    lib.gqa_decode_int8_masked.restype = ctypes.c_int
    lib.gqa_probe_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P]
    lib.gqa_probe_mfma_peak.restype = ctypes.c_int
    lib.gqa_probe_kv_stream.argtypes = [ctypes.c_int, ctypes.c_int, P, P, I64, P, ctypes.c_int, P, P]
    lib.gqa_probe_kv_stream.restype = ctypes.c_int
    lib.gqa_last_path.argtypes = []
    lib.gqa_last_path.restype = ctypes.c_int
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# The C entry points under their own names (ctypes arguments, status returned)
# ---------------------------------------------------------------------------
def gqa_plan(attrs: gqa_attrs, max_batch: int, max_q_len: int, max_kv_len: int):
    """Returns (status, plan handle or None)."""
    h = gqa_plan_t()
    st = load().gqa_plan(ctypes.byref(attrs), max_batch, max_q_len, max_kv_len, ctypes.byref(h))
    return st, (h if st == GQA_OK else None)


def gqa_plan_destroy(plan) -> None:
    load().gqa_plan_destroy(plan)


def gqa_workspace_size(plan) -> int:
    return int(load().gqa_workspace_size(plan))


def gqa_prefill(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink, workspace, ws_bytes,
                stream) -> int:
    return load().gqa_prefill(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink,
                              workspace, ws_bytes, stream)


def gqa_append_kv(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache, seqlens_k, stream) -> int:
    return load().gqa_append_kv(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache,
                                seqlens_k, stream)


def gqa_decode(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, workspace,
               ws_bytes, stream) -> int:
    return load().gqa_decode(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                             head_sink, workspace, ws_bytes, stream)


def gqa_decode_noalloc(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink,
                       stream) -> int:
    return load().gqa_decode_noalloc(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                                     head_sink, stream)


def gqa_append_decode(plan, B, curr, capacity, q, k_new, v_new, k_cache, v_cache, out, seqlens_k, head_sink,
                      workspace, ws_bytes, stream) -> int:
    return load().gqa_append_decode(plan, B, curr, capacity, q, k_new, v_new, k_cache, v_cache, out,
                                    seqlens_k, head_sink, workspace, ws_bytes, stream)


def gqa_apply_rotary(plan, B, H, L, pos0, x, y, tables, stream) -> int:
    return load().gqa_apply_rotary(plan, B, H, L, pos0, x, y,
                                   None if tables is None else ctypes.byref(tables), stream)


def gqa_prefill_rotary(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink, tables, stream) -> int:
    return load().gqa_prefill_rotary(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink,
                                     None if tables is None else ctypes.byref(tables), stream)


def gqa_append_kv_rotary(plan, B, curr, capacity, q, q_rot, k_new, v_new, k_cache, v_cache,
                         seqlens_k, tables, stream) -> int:
    return load().gqa_append_kv_rotary(plan, B, curr, capacity, q, q_rot, k_new, v_new, k_cache,
                                       v_cache, seqlens_k,
                                       None if tables is None else ctypes.byref(tables), stream)


def gqa_prefill_masked(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink, mask, stream) -> int:
    return load().gqa_prefill_masked(plan, B, Lq, Lk, q, k, v, out, nonpad_kv_seqlen, head_sink,
                                     None if mask is None else ctypes.byref(mask), stream)


def gqa_decode_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, mask,
                      workspace, ws_bytes, stream) -> int:
    return load().gqa_decode_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                                    head_sink, None if mask is None else ctypes.byref(mask),
                                    workspace, ws_bytes, stream)


def gqa_append_kv_fp8(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache, seqlens_k, k_scale,
                      v_scale, stream) -> int:
    return load().gqa_append_kv_fp8(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache,
                                    seqlens_k, k_scale, v_scale, stream)


def gqa_decode_fp8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scale,
                   v_scale, workspace, ws_bytes, stream) -> int:
    return load().gqa_decode_fp8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                                 head_sink, k_scale, v_scale, workspace, ws_bytes, stream)


def gqa_decode_fp8_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scale,
                          v_scale, mask, workspace, ws_bytes, stream) -> int:
    return load().gqa_decode_fp8_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                                        head_sink, k_scale, v_scale,
                                        None if mask is None else ctypes.byref(mask),
                                        workspace, ws_bytes, stream)


GQA_PATH_NONE, GQA_PATH_MATRIX_PREFILL, GQA_PATH_MATRIX_DECODE, GQA_PATH_STREAMING = 0, 1, 2, 3
PATH_NAMES = {0: "none", 1: "matrix_prefill", 2: "matrix_decode", 3: "streaming"}


def gqa_last_path() -> int:
    return int(load().gqa_last_path())


def gqa_append_kv_int8(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache, seqlens_k, k_scales, v_scales,
                       stream) -> int:
    return load().gqa_append_kv_int8(plan, B, curr, capacity, k_new, v_new, k_cache, v_cache, seqlens_k,
                                     k_scales, v_scales, stream)


def gqa_decode_int8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scales, v_scales,
                    workspace, ws_bytes, stream) -> int:
    return load().gqa_decode_int8(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink,
                                  k_scales, v_scales, workspace, ws_bytes, stream)


def gqa_decode_int8_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k, head_sink, k_scales,
                           v_scales, mask, workspace, ws_bytes, stream) -> int:
    return load().gqa_decode_int8_masked(plan, B, curr, capacity, q, k_cache, v_cache, out, seqlens_k,
                                         head_sink, k_scales, v_scales,
                                         None if mask is None else ctypes.byref(mask),
                                         workspace, ws_bytes, stream)


def gqa_probe_mfma_peak(blocks, iters, stamps, sink, stream) -> int:
    """Measurement aid (include/gqa_probe.h): back-to-back bf16 MFMAs with
    shader-clock and 100 MHz stamps per wave."""
    return load().gqa_probe_mfma_peak(blocks, iters, stamps, sink, stream)


def gqa_probe_kv_stream(grid, row_bytes, k, v, kv_bytes, unit_off, units, sink, stream) -> int:
    """Measurement aid (include/gqa_probe.h): K/V units of 16 rows of
    row_bytes streamed through the decode's loading scheme with no attention
    work."""
    return load().gqa_probe_kv_stream(grid, row_bytes, k, v, kv_bytes, unit_off, units, sink, stream)


def gqa_last_error() -> str:
    return load().gqa_last_error().decode()


# ---------------------------------------------------------------------------
# torch-tensor convenience layer
# ---------------------------------------------------------------------------
class GQAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != GQA_OK:
        raise GQAError(status, gqa_last_error())


def tensor_view(t, heads: Optional[int] = None) -> gqa_tensor:
    """gqa_tensor for a [B, H, L, D] tensor, or a [B, L, H*D] tensor with ``heads``."""
    if t.dim() == 4:
        sb, sh, ss, sd = t.stride()
    elif t.dim() == 3:
        if heads is None:
            raise ValueError("a [B, L, H*D] tensor needs the head count")
        sb, ss, sd = t.stride()
        sh = t.shape[2] // heads
    else:
        raise ValueError("expected a 4-D [B,H,L,D] or 3-D [B,L,H*D] tensor")
    if sd != 1:
        raise ValueError("the head dimension must be contiguous")
    return gqa_tensor(t.data_ptr(), sb, sh, ss)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


_TORCH_CODE = None


def _dtype_code(t):
    import torch
    global _TORCH_CODE
    if _TORCH_CODE is None:
        _TORCH_CODE = {torch.float32: GQA_F32, torch.float16: GQA_F16, torch.bfloat16: GQA_BF16}
    return _TORCH_CODE[t.dtype]


def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def _aux(name, t, dtype, n):
    """An optional per-batch or per-head array: dtype and at least n elements."""
    if t is None:
        return
    _need(t.dtype == dtype, f"{name} must be {dtype} (got {t.dtype})", TypeError)
    _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(t.numel() >= n, f"{name} needs at least {n} elements (got {t.numel()})")


def _same_device(ref, **ts):
    """Every tensor on ref's device, which must be a GPU: the library reads
    them as device pointers."""
    _need(ref.device.type == "cuda", f"tensors must be on a GPU (got {ref.device})")
    for name, t in ts.items():
        if t is not None:
            _need(t.device == ref.device, f"{name} is on {t.device}, not on {ref.device}")


class Plan:
    """An immutable attention plan (``gqa_plan``) driven with torch tensors.

    Every call checks its tensors' shapes against the plan (head counts, head
    size), the dtypes and lengths of the per-batch and per-head arrays
    (seqlens_k int32 [B], nonpad_kv_seqlen int64 [B], head_sink float32 [Hq])
    and that all of them live on the GPU of q, before any pointer reaches the
    library; a mismatch raises ValueError or TypeError.
    """

    def __init__(self, num_heads: int, kv_num_heads: int, head_size: int, *, dtype: str,
                 scale: float = 0.0, local_window_size: int = -1, softcap: float = 0.0,
                 smooth_softmax: bool = False, use_head_sink: bool = False,
                 is_causal: bool = True, rolling_cache: bool = False, max_batch: int = 1,
                 max_q_len: int = 1, max_kv_len: int = 1):
        self.attrs = gqa_attrs(num_heads, kv_num_heads, head_size, scale, local_window_size,
                               softcap, int(smooth_softmax), int(use_head_sink), int(is_causal),
                               DTYPE_CODES[dtype], int(rolling_cache))
        self.dtype = dtype
        self.num_heads, self.kv_num_heads, self.head_size = num_heads, kv_num_heads, head_size
        self._h = None
        st, h = gqa_plan(self.attrs, max_batch, max_q_len, max_kv_len)
        check(st)
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.gqa_plan_destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def workspace_size(self) -> int:
        return gqa_workspace_size(self._h)

    def new_workspace(self, device="cuda"):
        """A decode workspace; zero-filled, as the C ABI requires before first use."""
        import torch
        return torch.zeros(max(16, self.workspace_size()), dtype=torch.uint8, device=device)

    def _check_dtype(self, *ts):
        want = DTYPE_CODES[self.dtype]
        for t in ts:
            if t is not None and _dtype_code(t) != want:
                raise TypeError(f"tensor dtype {t.dtype} does not match the plan's {self.dtype}")

    def _rows(self, name, t, heads, layout="bhsd"):
        """(B, L) of a [B, H, L, D] (or [B, L, H*D]) tensor with the plan's head
        count and head size."""
        if layout == "bhsd":
            _need(t.dim() == 4, f"{name} must be 4-D [B, H, L, D]")
            _need(t.shape[1] == heads and t.shape[3] == self.head_size,
                  f"{name} has shape {tuple(t.shape)}: expected [B, {heads}, L, {self.head_size}]")
            return t.shape[0], t.shape[2]
        _need(t.dim() == 3, f"{name} must be 3-D [B, L, H*D]")
        _need(t.shape[2] == heads * self.head_size,
              f"{name} has shape {tuple(t.shape)}: expected [B, L, {heads * self.head_size}]")
        return t.shape[0], t.shape[1]

    def _caches(self, B, k_cache, v_cache, elem=None):
        """Capacity of a [>= B, Hkv, capacity, D] cache pair."""
        Bk, cap = self._rows("k_cache", k_cache, self.kv_num_heads)
        _need(tuple(v_cache.shape) == tuple(k_cache.shape), "k_cache and v_cache differ in shape")
        _need(Bk >= B, f"the caches hold {Bk} batches, fewer than B = {B}")
        if elem is not None:
            _need(k_cache.dtype == elem and v_cache.dtype == elem, f"caches must be {elem}", TypeError)
        return cap

    def _workspace(self, ws):
        _need(ws.is_contiguous(), "workspace must be contiguous")
        _need(ws.numel() * ws.element_size() >= self.workspace_size(),
              f"workspace of {self.workspace_size()} bytes needed")

    def mask_view(self, mask, B, Lq, Lk) -> gqa_mask:
        """gqa_mask for a bool (True attends) or float32 (additive) tensor
        broadcastable to [B, Hq, Lq, Lk]."""
        import torch
        if mask.dim() != 4:
            raise ValueError("a mask is 4-D, broadcastable to [B, Hq, Lq, Lk]")
        m = mask.expand(B, self.num_heads, Lq, Lk)
        if m.stride(3) != 1 and Lk > 1:
            raise ValueError("the mask's key dimension must be contiguous")
        if mask.dtype == torch.bool:
            kind = GQA_MASK_BOOL
        elif mask.dtype == torch.float32:
            kind = GQA_MASK_ADDITIVE
        else:
            raise TypeError("a mask is bool (True attends) or float32 (additive)")
        return gqa_mask(m.data_ptr(), m.stride(0), m.stride(1), m.stride(2), kind)

    def prefill(self, q, k, v, out=None, *, nonpad_kv_seqlen=None, head_sink=None,
                layout="bhsd", mask=None, stream=None):
        """q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] (layout "bhsd") or [B,L,H*D] ("bshd").
        ``mask``: bool or float32, broadcastable to [B, Hq, Lq, Lk]."""
        import torch
        self._check_dtype(q, k, v, out)
        B, Lq = self._rows("q", q, self.num_heads, layout)
        Bk, Lk = self._rows("k", k, self.kv_num_heads, layout)
        _need(tuple(v.shape) == tuple(k.shape), "k and v differ in shape")
        _need(Bk == B, f"q has {B} batches, k has {Bk}")
        _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
        _aux("nonpad_kv_seqlen", nonpad_kv_seqlen, torch.int64, B)
        _aux("head_sink", head_sink, torch.float32, self.num_heads)
        _same_device(q, k=k, v=v, out=out, nonpad_kv_seqlen=nonpad_kv_seqlen, head_sink=head_sink,
                     mask=mask)
        if out is None:
            out = torch.empty_like(q)
        if layout == "bhsd":
            B, _, Lq, _ = q.shape
            Lk = k.shape[2]
            qv, kv_, vv, ov = (tensor_view(x) for x in (q, k, v, out))
        else:
            B, Lq, _ = q.shape
            Lk = k.shape[1]
            qv, ov = tensor_view(q, self.num_heads), tensor_view(out, self.num_heads)
            kv_, vv = tensor_view(k, self.kv_num_heads), tensor_view(v, self.kv_num_heads)
        if mask is not None:
            check(gqa_prefill_masked(self._h, B, Lq, Lk, qv, kv_, vv, ov, _ptr(nonpad_kv_seqlen),
                                     _ptr(head_sink), self.mask_view(mask, B, Lq, Lk),
                                     _stream(stream)))
            return out
        check(gqa_prefill(self._h, B, Lq, Lk, qv, kv_, vv, ov, _ptr(nonpad_kv_seqlen),
                          _ptr(head_sink), None, 0, _stream(stream)))
        return out

    def append_kv(self, k_new, v_new, k_cache, v_cache, seqlens_k, *, stream=None):
        import torch
        self._check_dtype(k_new, v_new, k_cache, v_cache)
        B, curr = self._rows("k_new", k_new, self.kv_num_heads)
        _need(tuple(v_new.shape) == tuple(k_new.shape), "k_new and v_new differ in shape")
        self._caches(B, k_cache, v_cache)
        _need(seqlens_k is not None, "seqlens_k is required")
        _aux("seqlens_k", seqlens_k, torch.int32, B)
        _same_device(k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, seqlens_k=seqlens_k)
        check(gqa_append_kv(self._h, B, curr, k_cache.shape[2], tensor_view(k_new),
                            tensor_view(v_new), tensor_view(k_cache), tensor_view(v_cache),
                            _ptr(seqlens_k), _stream(stream)))

    def decode(self, q, k_cache, v_cache, seqlens_k, out=None, *, head_sink=None,
               workspace=None, mask=None, stream=None):
        """``mask``: bool or float32, broadcastable to [B, Hq, curr, capacity]."""
        import torch
        self._check_dtype(q, k_cache, v_cache, out)
        self._decode_args(q, k_cache, v_cache, seqlens_k, out, head_sink, workspace, mask)
        if out is None:
            out = torch.empty_like(q)
        if mask is not None:
            B, _, curr, _ = q.shape
            if workspace is None:
                workspace = self.new_workspace(q.device)
            check(gqa_decode_masked(self._h, B, curr, k_cache.shape[2], tensor_view(q),
                                    tensor_view(k_cache), tensor_view(v_cache), tensor_view(out),
                                    _ptr(seqlens_k), _ptr(head_sink),
                                    self.mask_view(mask, B, curr, k_cache.shape[2]),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))
            return out
        if workspace is None:
            workspace = self.new_workspace(q.device)
        B, _, curr, _ = q.shape
        check(gqa_decode(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                         tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream(stream)))
        return out

    def _decode_args(self, q, k_cache, v_cache, seqlens_k, out, head_sink, workspace, mask, elem=None):
        import torch
        B, _ = self._rows("q", q, self.num_heads)
        self._caches(B, k_cache, v_cache, elem)
        _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
        _need(seqlens_k is not None, "seqlens_k is required")
        _aux("seqlens_k", seqlens_k, torch.int32, B)
        _aux("head_sink", head_sink, torch.float32, self.num_heads)
        if workspace is not None:
            self._workspace(workspace)
        _same_device(q, k_cache=k_cache, v_cache=v_cache, seqlens_k=seqlens_k, out=out,
                     head_sink=head_sink, workspace=workspace, mask=mask)

    def append_decode(self, q, k_new, v_new, k_cache, v_cache, seqlens_k, out=None, *, head_sink=None,
                      workspace=None, stream=None):
        """One decode step (gqa_append_decode): append_kv then decode, in one
        launch on the matrix-core decode."""
        import torch
        self._check_dtype(q, k_new, v_new, k_cache, v_cache, out)
        self._decode_args(q, k_cache, v_cache, seqlens_k, out, head_sink, workspace, None)
        Bq, curr = self._rows("q", q, self.num_heads)
        B, curr_n = self._rows("k_new", k_new, self.kv_num_heads)
        _need((Bq, curr) == (B, curr_n), "q and k_new differ in batch or step length")
        _need(tuple(v_new.shape) == tuple(k_new.shape), "k_new and v_new differ in shape")
        _same_device(q, k_new=k_new, v_new=v_new)
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.device)
        check(gqa_append_decode(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_new),
                                tensor_view(v_new), tensor_view(k_cache), tensor_view(v_cache), tensor_view(out),
                                _ptr(seqlens_k), _ptr(head_sink), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
        return out

    def decode_noalloc(self, q, k_cache, v_cache, seqlens_k, out=None, *, head_sink=None, stream=None):
        """gqa_decode_noalloc: the decode with the library's static scratch
        instead of a workspace (no device allocation by the library; out is
        allocated here when not given)."""
        import torch
        self._check_dtype(q, k_cache, v_cache, out)
        self._decode_args(q, k_cache, v_cache, seqlens_k, out, head_sink, None, None)
        if out is None:
            out = torch.empty_like(q)
        B, _, curr, _ = q.shape
        check(gqa_decode_noalloc(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                                 tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                                 _stream(stream)))
        return out

    @staticmethod
    def _tables(cos, sin):
        import torch
        for t_ in (cos, sin):
            if t_.dtype != torch.float32 or t_.dim() != 2 or not t_.is_contiguous():
                raise ValueError("rotary tables must be contiguous float32 [max_pos, D/2]")
        if cos.shape != sin.shape:
            raise ValueError("cos and sin tables differ in shape")
        return gqa_rotary_tables(cos.data_ptr(), sin.data_ptr(), cos.shape[0])

    def apply_rotary(self, x, pos0, cos, sin, out=None, *, stream=None):
        """Rotary embedding of x [B, H, L, D] at positions pos0 + l (out may be x)."""
        import torch
        self._check_dtype(x, out)
        _need(x.dim() == 4 and x.shape[3] == self.head_size, f"x must be [B, H, L, {self.head_size}]")
        _need(out is None or tuple(out.shape) == tuple(x.shape), "out must have x's shape")
        if cos.shape[1] * 2 != self.head_size:
            raise ValueError("rotary tables need head_size / 2 columns")
        _same_device(x, out=out, cos=cos, sin=sin)
        if out is None:
            out = torch.empty_like(x)
        B, H, L, _ = x.shape
        check(gqa_apply_rotary(self._h, B, H, L, pos0, tensor_view(x), tensor_view(out),
                               self._tables(cos, sin), _stream(stream)))
        return out

    def prefill_rotary(self, q, k, v, cos, sin, out=None, *, nonpad_kv_seqlen=None, head_sink=None, stream=None):
        """gqa_prefill_rotary: q [B, Hq, Lq, D] not yet turned (turned in the
        prefill at positions Lk - Lq + i), k [B, Hkv, Lk, D] already turned."""
        import torch
        self._check_dtype(q, k, v, out)
        B, Lq = self._rows("q", q, self.num_heads)
        Bk, Lk = self._rows("k", k, self.kv_num_heads)
        _need(tuple(v.shape) == tuple(k.shape), "k and v differ in shape")
        _need(Bk == B, f"q has {B} batches, k has {Bk}")
        _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
        _aux("nonpad_kv_seqlen", nonpad_kv_seqlen, torch.int64, B)
        _aux("head_sink", head_sink, torch.float32, self.num_heads)
        if cos.shape[1] * 2 != self.head_size:
            raise ValueError("rotary tables need head_size / 2 columns")
        _same_device(q, k=k, v=v, out=out, nonpad_kv_seqlen=nonpad_kv_seqlen, head_sink=head_sink,
                     cos=cos, sin=sin)
        if out is None:
            out = torch.empty_like(q)
        check(gqa_prefill_rotary(self._h, B, Lq, Lk, tensor_view(q), tensor_view(k), tensor_view(v),
                                 tensor_view(out), _ptr(nonpad_kv_seqlen), _ptr(head_sink),
                                 self._tables(cos, sin), _stream(stream)))
        return out

    def append_kv_rotary(self, q, k_new, v_new, k_cache, v_cache, seqlens_k, cos, sin,
                         q_rot=None, *, stream=None):
        """One decode step's append with rotary; returns the rotated q (q_rot may be q)."""
        import torch
        self._check_dtype(q, k_new, v_new, k_cache, v_cache, q_rot)
        Bq, curr_q = self._rows("q", q, self.num_heads)
        B, curr = self._rows("k_new", k_new, self.kv_num_heads)
        _need((Bq, curr_q) == (B, curr), "q and k_new differ in batch or step length")
        _need(tuple(v_new.shape) == tuple(k_new.shape), "k_new and v_new differ in shape")
        _need(q_rot is None or tuple(q_rot.shape) == tuple(q.shape), "q_rot must have q's shape")
        self._caches(B, k_cache, v_cache)
        _need(seqlens_k is not None, "seqlens_k is required")
        _aux("seqlens_k", seqlens_k, torch.int32, B)
        if cos.shape[1] * 2 != self.head_size:
            raise ValueError("rotary tables need head_size / 2 columns")
        _same_device(q, q_rot=q_rot, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                     seqlens_k=seqlens_k, cos=cos, sin=sin)
        if q_rot is None:
            q_rot = torch.empty_like(q)
        B, _, curr, _ = k_new.shape
        check(gqa_append_kv_rotary(self._h, B, curr, k_cache.shape[2], tensor_view(q),
                                   tensor_view(q_rot), tensor_view(k_new), tensor_view(v_new),
                                   tensor_view(k_cache), tensor_view(v_cache), _ptr(seqlens_k),
                                   self._tables(cos, sin), _stream(stream)))
        return q_rot

    # ---- FP8 (E4M3) KV caches: uint8 tensors of codes, per-tensor scales ----
    def append_kv_fp8(self, k_new, v_new, k_cache, v_cache, seqlens_k, k_scale, v_scale, *, stream=None):
        import torch
        self._check_dtype(k_new, v_new)
        if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
            raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
        B, curr = self._rows("k_new", k_new, self.kv_num_heads)
        _need(tuple(v_new.shape) == tuple(k_new.shape), "k_new and v_new differ in shape")
        self._caches(B, k_cache, v_cache)
        _need(seqlens_k is not None, "seqlens_k is required")
        _aux("seqlens_k", seqlens_k, torch.int32, B)
        _same_device(k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, seqlens_k=seqlens_k)
        check(gqa_append_kv_fp8(self._h, B, curr, k_cache.shape[2], tensor_view(k_new),
                                tensor_view(v_new), tensor_view(k_cache), tensor_view(v_cache),
                                _ptr(seqlens_k), float(k_scale), float(v_scale), _stream(stream)))

    # ---- INT8 KV caches: int8 tensors of codes, per-KV-head scales ----
    def _int8_args(self, k_cache, v_cache, k_scales, v_scales):
        import torch
        if k_cache.dtype != torch.int8 or v_cache.dtype != torch.int8:
            raise TypeError("INT8 caches are int8 tensors of codes")
        _aux("k_scales", k_scales, torch.float32, self.kv_num_heads)
        _aux("v_scales", v_scales, torch.float32, self.kv_num_heads)
        _need(k_scales is not None and v_scales is not None, "k_scales and v_scales are required")

    def append_kv_int8(self, k_new, v_new, k_cache, v_cache, seqlens_k, k_scales, v_scales, *, stream=None):
        import torch
        self._check_dtype(k_new, v_new)
        self._int8_args(k_cache, v_cache, k_scales, v_scales)
        B, curr = self._rows("k_new", k_new, self.kv_num_heads)
        _need(tuple(v_new.shape) == tuple(k_new.shape), "k_new and v_new differ in shape")
        self._caches(B, k_cache, v_cache)
        _need(seqlens_k is not None, "seqlens_k is required")
        _aux("seqlens_k", seqlens_k, torch.int32, B)
        _same_device(k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, seqlens_k=seqlens_k,
                     k_scales=k_scales, v_scales=v_scales)
        check(gqa_append_kv_int8(self._h, B, curr, k_cache.shape[2], tensor_view(k_new), tensor_view(v_new),
                                 tensor_view(k_cache), tensor_view(v_cache), _ptr(seqlens_k), _ptr(k_scales),
                                 _ptr(v_scales), _stream(stream)))

    def decode_int8(self, q, k_cache, v_cache, seqlens_k, k_scales, v_scales, out=None, *, head_sink=None,
                    workspace=None, mask=None, stream=None):
        """``mask``: bool or float32, broadcastable to [B, Hq, curr, capacity]."""
        import torch
        self._check_dtype(q, out)
        self._int8_args(k_cache, v_cache, k_scales, v_scales)
        self._decode_args(q, k_cache, v_cache, seqlens_k, out, head_sink, workspace, mask, torch.int8)
        _same_device(q, k_scales=k_scales, v_scales=v_scales)
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.device)
        B, _, curr, _ = q.shape
        if mask is not None:
            m = self.mask_view(mask, B, curr, k_cache.shape[2])
            check(gqa_decode_int8_masked(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                                         tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                                         _ptr(k_scales), _ptr(v_scales), m, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
            return out
        check(gqa_decode_int8(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                              tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                              _ptr(k_scales), _ptr(v_scales), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
        return out

    def decode_fp8(self, q, k_cache, v_cache, seqlens_k, k_scale, v_scale, out=None, *,
                   head_sink=None, workspace=None, mask=None, stream=None):
        """``mask``: bool or float32, broadcastable to [B, Hq, curr, capacity]."""
        import torch
        self._check_dtype(q, out)
        if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
            raise TypeError("FP8 caches are uint8 tensors of E4M3 codes")
        self._decode_args(q, k_cache, v_cache, seqlens_k, out, head_sink, workspace, mask, torch.uint8)
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.device)
        B, _, curr, _ = q.shape
        if mask is not None:
            m = self.mask_view(mask, B, curr, k_cache.shape[2])
            check(gqa_decode_fp8_masked(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                                        tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                                        float(k_scale), float(v_scale), m, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
            return out
        check(gqa_decode_fp8(self._h, B, curr, k_cache.shape[2], tensor_view(q), tensor_view(k_cache),
                             tensor_view(v_cache), tensor_view(out), _ptr(seqlens_k), _ptr(head_sink),
                             float(k_scale), float(v_scale), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
        return out
