"""The C-ABI library on the host: it loads, exports exactly what include/gqa.h
declares, and rejects every malformed call before touching a device.

None of these calls reaches a kernel launch (each fails validation first), so
they run without a GPU.
"""

import ctypes
import os
import re
import subprocess

import pytest

from windowed_gqa_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

FAKE = 1 << 20  # a 16-byte aligned non-NULL address; never dereferenced


def declared_functions():
    """Functions declared by every header under include/ (the attention ABI
    and the measurement probe)."""
    src = "".join(open(os.path.join(ROOT, "include", f)).read()
                  for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", src)))


def attrs(**kw):
    base = dict(num_heads=8, kv_num_heads=2, head_size=128, scale=0.0, local_window_size=-1,
                softcap=0.0, smooth_softmax=0, use_head_sink=0, is_causal=1, dtype=B.GQA_BF16)
    base.update(kw)
    return B.gqa_attrs(**base)


def plan(**kw):
    st, h = B.gqa_plan(attrs(**kw), 4, 16, 1024)
    assert st == B.GQA_OK, B.gqa_last_error()
    return h


def t(ptr=FAKE, sb=1024 * 128 * 8, sh=1024 * 128, ss=128):
    return B.gqa_tensor(ptr, sb, sh, ss)


def test_library_exports_exactly_the_header():
    lib = B.load()
    names = declared_functions()
    assert names == sorted(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines()
                      if l.split()[-2] in ("T", "W") and l.split()[-1].startswith("gqa_"))
    assert exported == names


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_heads=0), B.GQA_ERR_INVALID_ARG, "num_heads"),
    (dict(kv_num_heads=0), B.GQA_ERR_INVALID_ARG, "kv_num_heads"),
    (dict(num_heads=8, kv_num_heads=3), B.GQA_ERR_INVALID_ARG, "multiple"),
    (dict(head_size=100), B.GQA_ERR_UNSUPPORTED, "head_size"),
    (dict(head_size=512), B.GQA_ERR_UNSUPPORTED, "head_size"),
    (dict(scale=-1.0), B.GQA_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), B.GQA_ERR_INVALID_ARG, "scale"),
    (dict(local_window_size=0), B.GQA_ERR_INVALID_ARG, "local_window_size"),
    (dict(local_window_size=-2), B.GQA_ERR_INVALID_ARG, "local_window_size"),
    (dict(softcap=-1.0), B.GQA_ERR_INVALID_ARG, "softcap"),
    (dict(softcap=float("inf")), B.GQA_ERR_INVALID_ARG, "softcap"),
    (dict(smooth_softmax=2), B.GQA_ERR_INVALID_ARG, "smooth_softmax"),
    (dict(use_head_sink=5), B.GQA_ERR_INVALID_ARG, "use_head_sink"),
    (dict(is_causal=0, local_window_size=4), B.GQA_ERR_INVALID_ARG, "is_causal"),
    (dict(dtype=7), B.GQA_ERR_INVALID_ARG, "dtype"),
])
def test_plan_rejects_bad_attributes(kw, status, needle):
    st, h = B.gqa_plan(attrs(**kw), 4, 16, 1024)
    assert st == status and h is None
    assert needle in B.gqa_last_error()


def test_plan_rejects_bad_limits_and_null():
    assert B.gqa_plan(attrs(), 0, 16, 1024)[0] == B.GQA_ERR_INVALID_ARG
    assert B.gqa_plan(attrs(), 4, 16, 1 << 31)[0] == B.GQA_ERR_UNSUPPORTED
    lib = B.load()
    assert lib.gqa_plan(None, 4, 16, 1024, ctypes.byref(B.gqa_plan_t())) == B.GQA_ERR_INVALID_ARG
    assert "attrs" in B.gqa_last_error()


def test_workspace_size_and_destroy():
    h = plan()
    assert B.gqa_workspace_size(h) > 0
    B.gqa_plan_destroy(h)
    assert B.gqa_workspace_size(None) == 0
    B.gqa_plan_destroy(None)
    # fp32 runs the generic kernels, which need no workspace
    h = plan(dtype=B.GQA_F32)
    assert B.gqa_workspace_size(h) == 0
    B.gqa_plan_destroy(h)


def _prefill(h, Bn=2, Lq=8, Lk=8, q=None, k=None, v=None, o=None, nonpad=None, sink=None):
    return B.gqa_prefill(h, Bn, Lq, Lk, q or t(), k or t(), v or t(), o or t(), nonpad, sink,
                         None, 0, None)


def test_prefill_validation():
    h = plan()
    assert _prefill(None) == B.GQA_ERR_INVALID_ARG
    assert _prefill(h, Bn=-1) == B.GQA_ERR_INVALID_ARG
    assert _prefill(h, Bn=5) == B.GQA_ERR_CAPACITY and "max_batch" in B.gqa_last_error()
    assert _prefill(h, Lq=17) == B.GQA_ERR_CAPACITY and "max_q_len" in B.gqa_last_error()
    assert _prefill(h, Lk=1025) == B.GQA_ERR_CAPACITY and "max_kv_len" in B.gqa_last_error()
    assert _prefill(h, q=t(ptr=0)) == B.GQA_ERR_INVALID_ARG and "q.data" in B.gqa_last_error()
    assert _prefill(h, k=t(ptr=FAKE + 2)) == B.GQA_ERR_UNSUPPORTED and "aligned" in B.gqa_last_error()
    assert _prefill(h, v=t(ss=100)) == B.GQA_ERR_UNSUPPORTED and "multiples" in B.gqa_last_error()
    assert _prefill(h, o=t(sh=-128)) == B.GQA_ERR_INVALID_ARG and "negative" in B.gqa_last_error()
    assert _prefill(h, sink=ctypes.c_void_p(FAKE)) == B.GQA_ERR_INVALID_ARG
    assert "use_head_sink" in B.gqa_last_error()
    # empty work is a no-op that succeeds without touching the device
    assert _prefill(h, Bn=0) == B.GQA_OK
    assert _prefill(h, Lq=0) == B.GQA_OK
    hs = plan(use_head_sink=1)
    assert _prefill(hs) == B.GQA_ERR_INVALID_ARG and "head_sink is NULL" in B.gqa_last_error()


def test_append_validation():
    h = plan()
    s = ctypes.c_void_p(FAKE)
    def app(Bn=2, curr=1, cap=64, seq=s, **kw):
        return B.gqa_append_kv(h, Bn, curr, cap, kw.get("kn", t()), kw.get("vn", t()),
                               kw.get("kc", t()), kw.get("vc", t()), seq, None)
    assert app(curr=17) == B.GQA_ERR_CAPACITY
    assert app(cap=1025) == B.GQA_ERR_CAPACITY
    assert app(curr=8, cap=4) == B.GQA_ERR_CAPACITY and "capacity" in B.gqa_last_error()
    assert app(seq=None) == B.GQA_ERR_INVALID_ARG and "seqlens_k" in B.gqa_last_error()
    assert app(kc=t(ptr=0)) == B.GQA_ERR_INVALID_ARG and "k_cache" in B.gqa_last_error()
    assert app(Bn=0) == B.GQA_OK


def test_decode_validation():
    h = plan()
    ws = B.gqa_workspace_size(h)
    s = ctypes.c_void_p(FAKE)
    def dec(Bn=2, curr=1, cap=64, seq=s, wsp=FAKE, wsb=ws, sink=None):
        return B.gqa_decode(h, Bn, curr, cap, t(), t(), t(), t(), seq, sink,
                            ctypes.c_void_p(wsp) if wsp else None, wsb, None)
    assert dec(curr=17) == B.GQA_ERR_CAPACITY
    assert dec(seq=None) == B.GQA_ERR_INVALID_ARG
    assert dec(wsp=0) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    assert dec(wsb=16) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    assert dec(wsp=FAKE + 8) == B.GQA_ERR_INVALID_ARG and "aligned" in B.gqa_last_error()
    assert dec(sink=ctypes.c_void_p(FAKE)) == B.GQA_ERR_INVALID_ARG
    assert dec(curr=0) == B.GQA_OK


def test_append_decode_validation():
    """gqa_append_decode checks the arguments of both calls it stands for."""
    h = plan()
    ws = B.gqa_workspace_size(h)
    s = ctypes.c_void_p(FAKE)
    def ad(Bn=2, curr=1, cap=64, seq=s, kn=None, wsb=ws, sink=None):
        return B.gqa_append_decode(h, Bn, curr, cap, t(), kn or t(), t(), t(), t(), t(), seq, sink,
                                   ctypes.c_void_p(FAKE), wsb, None)
    assert ad(curr=17) == B.GQA_ERR_CAPACITY
    assert ad(curr=8, cap=4) == B.GQA_ERR_CAPACITY and "capacity" in B.gqa_last_error()
    assert ad(seq=None) == B.GQA_ERR_INVALID_ARG and "seqlens_k" in B.gqa_last_error()
    assert ad(kn=t(ptr=0)) == B.GQA_ERR_INVALID_ARG and "k_new" in B.gqa_last_error()
    assert ad(wsb=16) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    assert ad(sink=ctypes.c_void_p(FAKE)) == B.GQA_ERR_INVALID_ARG
    assert ad(Bn=0) == B.GQA_OK


def test_decode_noalloc_validation():
    """gqa_decode_noalloc checks its arguments like gqa_decode, before it
    looks up its scratch array or launches anything."""
    h = plan()
    s = ctypes.c_void_p(FAKE)
    def dec(hh=h, Bn=2, curr=1, cap=64, seq=s, sink=None, q=None):
        return B.gqa_decode_noalloc(hh, Bn, curr, cap, q or t(), t(), t(), t(), seq, sink, None)
    assert dec(hh=None) == B.GQA_ERR_INVALID_ARG and "plan" in B.gqa_last_error()
    assert dec(Bn=5) == B.GQA_ERR_CAPACITY and "max_batch" in B.gqa_last_error()
    assert dec(curr=17) == B.GQA_ERR_CAPACITY
    assert dec(curr=8, cap=4) == B.GQA_ERR_CAPACITY and "capacity" in B.gqa_last_error()
    assert dec(seq=None) == B.GQA_ERR_INVALID_ARG and "seqlens_k" in B.gqa_last_error()
    assert dec(sink=ctypes.c_void_p(FAKE)) == B.GQA_ERR_INVALID_ARG and "use_head_sink" in B.gqa_last_error()
    assert dec(q=t(ptr=FAKE + 2)) == B.GQA_ERR_UNSUPPORTED and "aligned" in B.gqa_last_error()
    assert dec(Bn=0) == B.GQA_OK and dec(curr=0) == B.GQA_OK
    hr = plan(rolling_cache=1, local_window_size=100)
    assert dec(hh=hr, curr=4, cap=102) == B.GQA_ERR_CAPACITY and "rolling" in B.gqa_last_error()


def test_rotary_validation():
    h = plan()
    tab = B.gqa_rotary_tables(FAKE, FAKE, 64)
    s = ctypes.c_void_p(FAKE)
    def app(Bn=2, curr=1, cap=64, seq=s, tables=tab, **kw):
        return B.gqa_append_kv_rotary(h, Bn, curr, cap, kw.get("q", t()), kw.get("qr", t()),
                                      t(), t(), t(), t(), seq, tables, None)
    def rot(Bn=2, H=8, L=8, pos0=0, tables=tab, **kw):
        return B.gqa_apply_rotary(h, Bn, H, L, pos0, kw.get("x", t()), kw.get("y", t()), tables, None)
    assert app(tables=None) == B.GQA_ERR_INVALID_ARG and "tables" in B.gqa_last_error()
    assert app(tables=B.gqa_rotary_tables(0, FAKE, 64)) == B.GQA_ERR_INVALID_ARG
    assert app(tables=B.gqa_rotary_tables(FAKE + 4, FAKE, 64)) == B.GQA_ERR_UNSUPPORTED
    # every cache slot is a position: the tables must cover the capacity
    assert app(cap=65) == B.GQA_ERR_CAPACITY and "rotary tables" in B.gqa_last_error()
    assert app(curr=17) == B.GQA_ERR_CAPACITY
    assert app(seq=None) == B.GQA_ERR_INVALID_ARG and "seqlens_k" in B.gqa_last_error()
    assert app(qr=t(ptr=0)) == B.GQA_ERR_INVALID_ARG and "q_rot" in B.gqa_last_error()
    assert app(Bn=0) == B.GQA_OK
    assert rot(L=60, pos0=5) == B.GQA_ERR_CAPACITY and "rotary tables" in B.gqa_last_error()
    assert rot(pos0=-1) == B.GQA_ERR_INVALID_ARG
    assert rot(x=t(ptr=FAKE + 2)) == B.GQA_ERR_UNSUPPORTED and "aligned" in B.gqa_last_error()
    assert rot(tables=B.gqa_rotary_tables(FAKE, FAKE, 0)) == B.GQA_ERR_INVALID_ARG
    assert rot(L=0) == B.GQA_OK and rot(H=0) == B.GQA_OK
    # prefill with Q turned inside: the tables cover positions 0 .. Lk - 1
    def pr(Lk=8, tables=tab, hh=h, Bn=2):
        return B.gqa_prefill_rotary(hh, Bn, 8, Lk, t(), t(), t(), t(), None, None, tables, None)
    assert pr(tables=None) == B.GQA_ERR_INVALID_ARG and "tables" in B.gqa_last_error()
    assert pr(Lk=65) == B.GQA_ERR_CAPACITY and "rotary tables" in B.gqa_last_error()
    st, hf = B.gqa_plan(attrs(dtype=B.GQA_F32), 4, 16, 1024)
    assert pr(hh=hf) == B.GQA_ERR_UNSUPPORTED and "gqa_apply_rotary" in B.gqa_last_error()
    assert pr(Bn=0) == B.GQA_OK


def test_rolling_cache_validation():
    st, _ = B.gqa_plan(attrs(rolling_cache=1), 4, 16, 1024)  # window off
    assert st == B.GQA_ERR_INVALID_ARG and "rolling_cache" in B.gqa_last_error()
    st, _ = B.gqa_plan(attrs(rolling_cache=2, local_window_size=8), 4, 16, 1024)
    assert st == B.GQA_ERR_INVALID_ARG
    h = plan(rolling_cache=1, local_window_size=100)
    s = ctypes.c_void_p(FAKE)
    ws = B.gqa_workspace_size(h)
    # the ring must hold W + curr - 1 keys: 100 + 4 - 1 = 103
    assert B.gqa_append_kv(h, 2, 4, 102, t(), t(), t(), t(), s, None) == B.GQA_ERR_CAPACITY
    assert "rolling" in B.gqa_last_error()
    assert B.gqa_decode(h, 2, 4, 102, t(), t(), t(), t(), s, None, ctypes.c_void_p(FAKE), ws,
                        None) == B.GQA_ERR_CAPACITY
    tab = B.gqa_rotary_tables(FAKE, FAKE, 64)
    assert B.gqa_append_kv_rotary(h, 2, 4, 102, t(), t(), t(), t(), t(), t(), s, tab,
                                  None) == B.GQA_ERR_CAPACITY
    # exactly enough passes validation (B = 0: nothing is launched)
    assert B.gqa_append_kv(h, 0, 4, 103, t(), t(), t(), t(), s, None) == B.GQA_OK
    assert B.gqa_decode(h, 0, 4, 103, t(), t(), t(), t(), s, None, ctypes.c_void_p(FAKE), ws,
                        None) == B.GQA_OK
    # a rolling cache's positions pass the capacity: the tables need not cover it
    assert B.gqa_append_kv_rotary(h, 0, 4, 103, t(), t(), t(), t(), t(), t(), s, tab,
                                  None) == B.GQA_OK


def test_mask_validation():
    h = plan()
    s = ctypes.c_void_p(FAKE)
    ok = B.gqa_mask(FAKE, 0, 0, 1024, B.GQA_MASK_BOOL)
    def pf(mask, Bn=2, **kw):
        return B.gqa_prefill_masked(h, Bn, 8, 8, t(), t(), t(), t(), None, None, mask, None)
    ws = B.gqa_workspace_size(h)
    def dc(mask, Bn=2, hh=h, wsp=None, wsb=0):
        return B.gqa_decode_masked(hh, Bn, 1, 64, t(), t(), t(), t(), s, None, mask,
                                   ctypes.c_void_p(wsp) if wsp else None, wsb, None)
    assert pf(None) == B.GQA_ERR_INVALID_ARG and "mask" in B.gqa_last_error()
    assert pf(B.gqa_mask(0, 0, 0, 8, 1)) == B.GQA_ERR_INVALID_ARG and "mask.data" in B.gqa_last_error()
    assert pf(B.gqa_mask(FAKE, 0, 0, 8, 3)) == B.GQA_ERR_INVALID_ARG and "kind" in B.gqa_last_error()
    assert pf(B.gqa_mask(FAKE, -1, 0, 8, 1)) == B.GQA_ERR_INVALID_ARG and "negative" in B.gqa_last_error()
    assert pf(B.gqa_mask(FAKE + 2, 0, 0, 8, 2)) == B.GQA_ERR_UNSUPPORTED and "aligned" in B.gqa_last_error()
    assert pf(ok, Bn=5) == B.GQA_ERR_CAPACITY
    assert pf(ok, Bn=0) == B.GQA_OK
    assert dc(None) == B.GQA_ERR_INVALID_ARG
    assert dc(ok, Bn=0) == B.GQA_OK
    # the matrix-core path checks its workspace like gqa_decode
    ok4 = B.gqa_mask(FAKE, 0, 0, 1024, B.GQA_MASK_BOOL)
    assert dc(ok4, wsp=FAKE, wsb=16) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    assert dc(ok4, wsp=FAKE + 8, wsb=ws) == B.GQA_ERR_INVALID_ARG and "aligned" in B.gqa_last_error()
    hr = plan(rolling_cache=1, local_window_size=8)
    assert dc(ok, hh=hr) == B.GQA_ERR_UNSUPPORTED and "rolling" in B.gqa_last_error()


def test_fp8_validation():
    h = plan()
    s = ctypes.c_void_p(FAKE)
    ws = B.gqa_workspace_size(h)
    c8 = B.gqa_tensor(FAKE, 1024 * 128 * 2, 1024 * 128, 128)  # byte strides of a uint8 cache
    def app(ks=1.0, vs=1.0, kc=c8, Bn=2):
        return B.gqa_append_kv_fp8(h, Bn, 1, 64, t(), t(), kc, c8, s, ks, vs, None)
    def dec(ks=1.0, vs=1.0, hh=h, wsp=FAKE, kc=c8, Bn=2):
        return B.gqa_decode_fp8(hh, Bn, 1, 64, t(), kc, c8, t(), s, None, ks, vs,
                                ctypes.c_void_p(wsp) if wsp else None, ws, None)
    assert app(ks=0.0) == B.GQA_ERR_INVALID_ARG and "scale" in B.gqa_last_error()
    assert app(vs=float("inf")) == B.GQA_ERR_INVALID_ARG
    assert app(kc=B.gqa_tensor(FAKE, 1024 * 128 * 2, 1024 * 128, 100)) == B.GQA_ERR_UNSUPPORTED
    assert app(Bn=0) == B.GQA_OK
    assert dec(ks=-1.0) == B.GQA_ERR_INVALID_ARG
    assert dec(wsp=0) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    assert dec(Bn=0) == B.GQA_OK
    st, h96 = B.gqa_plan(attrs(head_size=96), 4, 16, 1024)
    assert st == B.GQA_OK
    assert dec(hh=h96) == B.GQA_ERR_UNSUPPORTED and "FP8" in B.gqa_last_error()
    st, hf = B.gqa_plan(attrs(dtype=B.GQA_F32), 4, 16, 1024)
    assert dec(hh=hf) == B.GQA_ERR_UNSUPPORTED

    # with a caller mask: FP8 caches have only the matrix-core decode
    def dm(mask, hh=h, Bn=2, ks=1.0):
        return B.gqa_decode_fp8_masked(hh, Bn, 1, 64, t(), c8, c8, t(), s, None, ks, 1.0, mask,
                                       ctypes.c_void_p(FAKE), ws, None)
    ok = B.gqa_mask(FAKE, 0, 0, 64, B.GQA_MASK_BOOL)
    assert dm(None) == B.GQA_ERR_INVALID_ARG and "mask" in B.gqa_last_error()
    assert dm(ok, ks=0.0) == B.GQA_ERR_INVALID_ARG and "scale" in B.gqa_last_error()
    assert dm(B.gqa_mask(FAKE + 2, 0, 0, 64, B.GQA_MASK_BOOL)) == B.GQA_ERR_UNSUPPORTED
    assert "FP8" in B.gqa_last_error()
    assert dm(B.gqa_mask(FAKE, 0, 0, 66, B.GQA_MASK_ADDITIVE)) == B.GQA_ERR_UNSUPPORTED
    assert dm(B.gqa_mask(FAKE, 0, 0, 64, 3)) == B.GQA_ERR_INVALID_ARG and "kind" in B.gqa_last_error()
    hr = plan(rolling_cache=1, local_window_size=8)
    assert dm(ok, hh=hr) == B.GQA_ERR_UNSUPPORTED and "rolling" in B.gqa_last_error()
    assert dm(ok, Bn=0) == B.GQA_OK


def test_int8_validation():
    h = plan()
    s = ctypes.c_void_p(FAKE)
    ws = B.gqa_workspace_size(h)
    c8 = B.gqa_tensor(FAKE, 1024 * 128 * 2, 1024 * 128, 128)
    sc = ctypes.c_void_p(FAKE)
    def app(ks=sc, Bn=2, kc=c8):
        return B.gqa_append_kv_int8(h, Bn, 1, 64, t(), t(), kc, c8, s, ks, sc, None)
    def dec(ks=sc, hh=h, wsp=FAKE, Bn=2):
        return B.gqa_decode_int8(hh, Bn, 1, 64, t(), c8, c8, t(), s, None, ks, sc,
                                 ctypes.c_void_p(wsp) if wsp else None, ws, None)
    assert app(ks=None) == B.GQA_ERR_INVALID_ARG and "scales" in B.gqa_last_error()
    assert app(kc=B.gqa_tensor(FAKE, 1024 * 128 * 2, 1024 * 128, 100)) == B.GQA_ERR_UNSUPPORTED
    assert app(Bn=0) == B.GQA_OK
    assert dec(ks=None) == B.GQA_ERR_INVALID_ARG
    assert dec(wsp=0) == B.GQA_ERR_INVALID_ARG and "workspace" in B.gqa_last_error()
    st, hf = B.gqa_plan(attrs(dtype=B.GQA_F32), 4, 16, 1024)
    assert dec(hh=hf) == B.GQA_ERR_UNSUPPORTED and "INT8" in B.gqa_last_error()
    assert dec(Bn=0) == B.GQA_OK

    # with a caller mask: INT8 caches have only the matrix-core decode
    def dm(mask, hh=h, Bn=2, ks=sc):
        return B.gqa_decode_int8_masked(hh, Bn, 1, 64, t(), c8, c8, t(), s, None, ks, sc, mask,
                                        ctypes.c_void_p(FAKE), ws, None)
    ok = B.gqa_mask(FAKE, 0, 0, 64, B.GQA_MASK_BOOL)
    assert dm(None) == B.GQA_ERR_INVALID_ARG and "mask" in B.gqa_last_error()
    assert dm(ok, ks=None) == B.GQA_ERR_INVALID_ARG and "scales" in B.gqa_last_error()
    assert dm(B.gqa_mask(FAKE + 2, 0, 0, 64, B.GQA_MASK_BOOL)) == B.GQA_ERR_UNSUPPORTED
    assert "INT8" in B.gqa_last_error()
    assert dm(B.gqa_mask(FAKE + 8, 0, 0, 64, B.GQA_MASK_ADDITIVE)) == B.GQA_ERR_UNSUPPORTED
    assert dm(B.gqa_mask(FAKE, 0, 0, 66, B.GQA_MASK_ADDITIVE)) == B.GQA_ERR_UNSUPPORTED
    assert dm(B.gqa_mask(FAKE, 0, 0, 64, 3)) == B.GQA_ERR_INVALID_ARG and "kind" in B.gqa_last_error()
    assert dm(ok, hh=hf) == B.GQA_ERR_UNSUPPORTED and "INT8" in B.gqa_last_error()
    hr = plan(rolling_cache=1, local_window_size=8)
    assert dm(ok, hh=hr) == B.GQA_ERR_UNSUPPORTED and "rolling" in B.gqa_last_error()
    assert dm(ok, Bn=0) == B.GQA_OK


def test_last_path_is_none_after_failed_or_empty_calls():
    h = plan()
    assert _prefill(h, Lq=17) == B.GQA_ERR_CAPACITY
    assert B.gqa_last_path() == B.GQA_PATH_NONE
    assert _prefill(h, Bn=0) == B.GQA_OK
    assert B.gqa_last_path() == B.GQA_PATH_NONE


def test_last_error_is_thread_local_and_specific():
    import threading
    B.gqa_plan(attrs(num_heads=0), 1, 1, 1)
    msg = []
    th = threading.Thread(target=lambda: msg.append(B.gqa_last_error()))
    th.start()
    th.join()
    assert msg == [""]
    assert "num_heads" in B.gqa_last_error()
