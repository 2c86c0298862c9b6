"""Pins of the float64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute by itself:
a brute-force restatement, a library routine that the special case reduces
to (torch's scaled_dot_product_attention in float64), an invariant the pages
state, a closed form, or a hand-worked example (tests/golden/).  The
mutation tests at the end plant plausible mistakes in a copy of the oracle
and check that some pin catches each one.
"""

import importlib.util
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch
from hypothesis import given, settings, HealthCheck, strategies as st

import oracle
from oracle import materialized as oracle_mod
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _interval_count(q_abs, valid, causal, window):
    """Allowed-key count of one row from the interval form of the rule
    (keys [max(0, p-W+1), min(p, valid-1)]), restated here independently of
    the oracle's elementwise predicate."""
    hi = min(q_abs, valid - 1) if causal else valid - 1
    lo = max(0, q_abs - window + 1) if window != -1 else 0
    return max(0, hi - lo + 1)


# --------------------------------------------------------------------------
# P-1: brute force on tiny shapes drawn by hypothesis, all features
# --------------------------------------------------------------------------
@st.composite
def tiny_case(draw):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 2))
    G = draw(st.integers(1, 3))
    D = draw(st.integers(1, 4))
    Lk = draw(st.integers(1, 10))
    Lq = draw(st.integers(1, 8))
    causal = draw(st.booleans())
    window = draw(st.sampled_from([-1, 1, 2, 3, 5, 12])) if causal else -1
    softcap = draw(st.sampled_from([0.0, 0.7, 3.0]))
    sink_mode = draw(st.sampled_from(["none", "smooth", "head"]))
    q_offset = [draw(st.integers(-3, Lk)) for _ in range(B)]
    valid = [draw(st.integers(0, Lk)) for _ in range(B)]
    scale = draw(st.sampled_from([0.3, 1.0, 1.7]))
    seed = draw(st.integers(0, 2**31 - 1))
    return dict(B=B, Hkv=Hkv, G=G, D=D, Lk=Lk, Lq=Lq, causal=causal, window=window,
                softcap=softcap, sink_mode=sink_mode, q_offset=q_offset, valid=valid,
                scale=scale, seed=seed)


@settings(max_examples=250, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(tiny_case())
def test_p1_brute_force_agrees(c):
    rng = np.random.default_rng(c["seed"])
    Hq = c["Hkv"] * c["G"]
    q = _rand(rng, c["B"], Hq, c["Lq"], c["D"])
    k = _rand(rng, c["B"], c["Hkv"], c["Lk"], c["D"])
    v = _rand(rng, c["B"], c["Hkv"], c["Lk"], c["D"])
    head = rng.standard_normal(Hq)
    sink = oracle.sink_logits(Hq, c["sink_mode"] == "smooth",
                              head if c["sink_mode"] == "head" else None)
    kw = dict(scale=c["scale"], causal=c["causal"], window=c["window"],
              softcap=c["softcap"], sink=sink)
    got = oracle.attention(q, k, v, c["q_offset"], c["valid"], **kw)
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), c["q_offset"],
                                    c["valid"], **kw))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P-2: reduction to torch's scaled_dot_product_attention (float64, CPU)
# --------------------------------------------------------------------------
def _sdpa_reference(q, k, v, q_offset, valid, scale, causal, window, sink):
    """SDPA over K/V repeated per query head; the sink is an appended zero
    key with a zero value whose additive mask entry is s_h."""
    B, Hq, Lq, D = q.shape
    G = Hq // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    Lk = k.shape[2]
    allowed = np.zeros((B, 1, Lq, Lk), dtype=bool)
    for b in range(B):
        for i in range(Lq):
            p = q_offset[b] + i
            for j in range(Lk):
                ok = j < valid[b]
                if causal:
                    ok = ok and j <= p
                if window != -1:
                    ok = ok and p - j < window
                allowed[b, 0, i, j] = ok
    bias = np.where(allowed, 0.0, -np.inf)
    bias = np.broadcast_to(bias, (B, Hq, Lq, Lk))
    if sink is not None:
        zeros = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
        kt = torch.cat([kt, zeros], dim=2)
        vt = torch.cat([vt, zeros], dim=2)
        col = np.broadcast_to(np.asarray(sink)[None, :, None, None], (B, Hq, Lq, 1))
        bias = np.concatenate([bias, col], axis=3)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=torch.from_numpy(np.ascontiguousarray(bias)),
        scale=scale)
    return out.numpy(), allowed[:, 0].any(axis=2)


@pytest.mark.parametrize("causal,window,sink_mode,nonpad", [
    (True, -1, "none", None),
    (True, 5, "none", None),
    (True, 1, "head", None),
    (True, 7, "smooth", (13, 9)),
    (False, -1, "head", (20, 3)),
    (True, 20, "head", (20, 17)),
])
def test_p2_matches_library_sdpa(causal, window, sink_mode, nonpad):
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, Lq, Lk = 2, 6, 2, 8, 11, 20
    q, k, v = _rand(rng, B, Hq, Lq, D), _rand(rng, B, Hkv, Lk, D), _rand(rng, B, Hkv, Lk, D)
    head = rng.standard_normal(Hq)
    sink = oracle.sink_logits(Hq, sink_mode == "smooth", head if sink_mode == "head" else None)
    valid = list(nonpad) if nonpad else [Lk] * B
    q_offset = [Lk - Lq] * B
    got = oracle.attention(q, k, v, q_offset, valid, scale=0.4, causal=causal,
                           window=window, sink=sink)
    want, has = _sdpa_reference(q, k, v, q_offset, valid, 0.4, causal, window, sink)
    has = np.broadcast_to(has[:, None, :], got.shape[:3])
    np.testing.assert_allclose(got[has], want[has], rtol=0, atol=1e-12)
    if sink is not None:
        # with a sink every row is defined for SDPA too (zero-value column)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_p2_plain_causal_is_torch_is_causal():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 3, 9, 5), _rand(rng, 1, 3, 9, 5), _rand(rng, 1, 3, 9, 5)
    got = oracle.prefill(q, k, v, scale=0.5)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        scale=0.5).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P-3 .. P-10: invariants
# --------------------------------------------------------------------------
def test_p3_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(3)
    B, Hkv, G, D, L = 2, 3, 4, 6, 17
    q, k, v = _rand(rng, B, Hkv * G, L, D), _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    sink = rng.standard_normal(Hkv * G)
    kw = dict(scale=0.3, window=5, head_sink=sink, softcap=2.0)
    a = oracle.prefill(q, k, v, **kw)
    b = oracle.prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), **kw)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_p4_wide_window_is_plain_causal(kind):
    rng = np.random.default_rng(4)
    if kind == "prefill":
        q, k, v = _rand(rng, 2, 4, 12, 4), _rand(rng, 2, 2, 12, 4), _rand(rng, 2, 2, 12, 4)
        a = oracle.prefill(q, k, v, scale=0.5, window=-1, nonpad_kv_seqlen=[12, 7])
        for W in (12, 13, 1000):
            b = oracle.prefill(q, k, v, scale=0.5, window=W, nonpad_kv_seqlen=[12, 7])
            np.testing.assert_array_equal(a, b)
    else:
        q = _rand(rng, 2, 4, 3, 4)
        kc, vc = _rand(rng, 2, 2, 16, 4), _rand(rng, 2, 2, 16, 4)
        s = [9, 15]
        a = oracle.decode(q, kc, vc, s, scale=0.5, window=-1)
        for W in (16, 40):
            np.testing.assert_array_equal(a, oracle.decode(q, kc, vc, s, scale=0.5, window=W))


@pytest.mark.parametrize("with_sink", [False, True])
def test_p5_window_one_is_self_only(with_sink):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, L = 2, 4, 2, 3, 9
    q, k, v = _rand(rng, B, Hq, L, D), _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    sink = rng.standard_normal(Hq) if with_sink else None
    nonpad = [9, 6]
    got = oracle.prefill(q, k, v, scale=0.7, window=1, head_sink=sink, nonpad_kv_seqlen=nonpad)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(L):
                if i >= nonpad[b]:
                    want = np.zeros(D)
                elif sink is None:
                    want = v[b, g, i]
                else:
                    x = 0.7 * float(q[b, h, i] @ k[b, g, i])
                    want = v[b, g, i] / (1.0 + math.exp(sink[h] - x))
                np.testing.assert_allclose(got[b, h, i], want, rtol=0, atol=1e-14)


def test_p6_zero_head_sink_is_smooth_softmax():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 4, 10, 4), _rand(rng, 1, 2, 10, 4), _rand(rng, 1, 2, 10, 4)
    a = oracle.prefill(q, k, v, scale=0.5, window=3, smooth_softmax=True)
    b = oracle.prefill(q, k, v, scale=0.5, window=3, head_sink=np.zeros(4))
    c = oracle.prefill(q, k, v, scale=0.5, window=3, smooth_softmax=True, head_sink=np.zeros(4))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)
    plain = oracle.prefill(q, k, v, scale=0.5, window=3)
    assert np.abs(plain - a).max() > 1e-3  # the sink really changes the result


def test_p7_single_key_sink_closed_form():
    rng = np.random.default_rng(71)
    for _ in range(20):
        q, k, v = _rand(rng, 1, 1, 1, 5), _rand(rng, 1, 1, 1, 5), _rand(rng, 1, 1, 1, 5)
        s = float(rng.standard_normal() * 3)
        got = oracle.prefill(q, k, v, scale=0.9, head_sink=[s])
        x = 0.9 * float(q[0, 0, 0] @ k[0, 0, 0])
        sig = 1.0 / (1.0 + math.exp(-(x - s)))
        np.testing.assert_allclose(got[0, 0, 0], sig * v[0, 0, 0], rtol=0, atol=1e-14)


def test_p8_fully_masked_rows_are_zero():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 2, 2, 6, 3), _rand(rng, 2, 1, 6, 3), _rand(rng, 2, 1, 6, 3)
    for sink in (None, np.array([2.0, -1.0])):
        out = oracle.prefill(q, k, v, scale=1.0, head_sink=sink, nonpad_kv_seqlen=[0, 6])
        assert np.all(out[0] == 0.0)
        assert np.all(np.isfinite(out))
    # more query rows than keys: rows at negative positions see nothing
    q2 = _rand(rng, 1, 2, 9, 3)
    out = oracle.prefill(q2, k[:1], v[:1], scale=1.0, head_sink=np.array([0.5, 0.5]))
    assert np.all(out[0, :, :3] == 0.0) and np.all(np.abs(out[0, :, 3:]).sum(-1) > 0)


def test_p8_large_gqa_shape_last_row_empty():
    """Keys 24576.. are padding and W = 8192: row 32767 of that batch sees no
    key (exact zero), row 32766 sees exactly key 24575."""
    rng = np.random.default_rng(88)
    L, D = 32768, 4
    q, k, v = _rand(rng, 1, 1, L, D), _rand(rng, 1, 1, L, D), _rand(rng, 1, 1, L, D)
    s = 0.3
    out = oracle.prefill(q, k, v, scale=0.5, window=8192, head_sink=[s],
                         nonpad_kv_seqlen=[24576], rows=[32766, 32767])
    assert np.all(out[0, 0, 1] == 0.0)
    x = 0.5 * float(q[0, 0, 32766] @ k[0, 0, 24575])
    want = v[0, 0, 24575] / (1.0 + math.exp(s - x))
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-14)


def test_p9_stale_and_padded_slots_never_matter():
    rng = np.random.default_rng(9)
    # decode: slots > seqlens_k are stale
    q = _rand(rng, 2, 4, 3, 4)
    kc, vc = _rand(rng, 2, 2, 20, 4), _rand(rng, 2, 2, 20, 4)
    s = np.array([8, 13])
    a = oracle.decode(q, kc, vc, s, scale=0.5, window=4, head_sink=np.ones(4))
    kp, vp = kc.copy(), vc.copy()
    for b in range(2):
        kp[b, :, s[b] + 1:] = np.nan
        vp[b, :, s[b] + 1:] = np.inf
    b_ = oracle.decode(q, kp, vp, s, scale=0.5, window=4, head_sink=np.ones(4))
    np.testing.assert_array_equal(a, b_)
    # prefill: slots >= nonpad are padding
    q, k, v = _rand(rng, 2, 2, 10, 4), _rand(rng, 2, 2, 10, 4), _rand(rng, 2, 2, 10, 4)
    a = oracle.prefill(q, k, v, scale=0.5, nonpad_kv_seqlen=[10, 4])
    k[1, :, 4:] = np.nan
    v[1, :, 4:] = np.nan
    np.testing.assert_array_equal(a, oracle.prefill(q, k, v, scale=0.5, nonpad_kv_seqlen=[10, 4]))


@pytest.mark.parametrize("curr,window", [(1, -1), (2, 3), (3, 1), (4, 6)])
def test_p10_decode_equals_prefill_tail(curr, window):
    rng = np.random.default_rng(10 + curr)
    P, cap, Hq, Hkv, D = 7, 16, 4, 2, 5
    total = P + curr
    q = _rand(rng, 1, Hq, total, D)
    k, v = _rand(rng, 1, Hkv, total, D), _rand(rng, 1, Hkv, total, D)
    sink = rng.standard_normal(Hq)
    full = oracle.prefill(q, k, v, scale=0.6, window=window, head_sink=sink, softcap=4.0)
    kc, vc = _rand(rng, 1, Hkv, cap, D), _rand(rng, 1, Hkv, cap, D)
    kc, vc = oracle.append_kv(kc, vc, k[:, :, :P], v[:, :, :P], [P - 1])
    kc, vc = oracle.append_kv(kc, vc, k[:, :, P:], v[:, :, P:], [total - 1])
    dec = oracle.decode(q[:, :, P:], kc, vc, [total - 1], scale=0.6, window=window,
                        head_sink=sink, softcap=4.0)
    np.testing.assert_allclose(dec, full[:, :, P:], rtol=0, atol=1e-13)


def test_append_kv_is_concatenation():
    rng = np.random.default_rng(11)
    kc, vc = _rand(rng, 2, 3, 10, 4), _rand(rng, 2, 3, 10, 4)
    kn, vn = _rand(rng, 2, 3, 2, 4), _rand(rng, 2, 3, 2, 4)
    k2, v2 = oracle.append_kv(kc, vc, kn, vn, [4, 9])
    np.testing.assert_array_equal(k2[0, :, 3:5], kn[0])
    np.testing.assert_array_equal(v2[1, :, 8:10], vn[1])
    np.testing.assert_array_equal(k2[0, :, :3], kc[0, :, :3])
    np.testing.assert_array_equal(k2[0, :, 5:], kc[0, :, 5:])
    with pytest.raises(ValueError):
        oracle.append_kv(kc, vc, kn, vn, [0, 9])  # total 1 < curr 2
    with pytest.raises(ValueError):
        oracle.append_kv(kc, vc, kn, vn, [4, 10])  # total 11 > capacity 10


# --------------------------------------------------------------------------
# P-11 .. P-13: probes with closed-form outputs
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal,window,nonpad,Lq,Lk", [
    (True, -1, None, 12, 12), (True, 3, None, 12, 12), (True, 5, (12, 7), 9, 12),
    (True, 1, None, 14, 10), (False, -1, (4, 12), 6, 12), (True, 64, (12, 0), 12, 12),
])
def test_p11_mask_probe(causal, window, nonpad, Lq, Lk):
    B, Hq, Hkv, D = 2, 2, 1, 12
    q = np.random.default_rng(111).standard_normal((B, Hq, Lq, D))
    k = np.zeros((B, Hkv, Lk, D))
    v = np.zeros((B, Hkv, Lk, D))
    probe = np.arange(D) % Lk
    for d in range(D):
        v[:, :, probe[d], d] = 1.0
    sink = np.array([0.0, 1.5])
    out = oracle.prefill(q, k, v, scale=1.0, causal=causal, window=window,
                         head_sink=sink, nonpad_kv_seqlen=nonpad)
    valid = nonpad if nonpad else (Lk, Lk)
    for b in range(B):
        for h in range(Hq):
            for i in range(Lq):
                p = Lk - Lq + i
                n = _interval_count(p, valid[b], causal, window)
                for d in range(D):
                    j = probe[d]
                    hi = min(p, valid[b] - 1) if causal else valid[b] - 1
                    lo = max(0, p - window + 1) if window != -1 else 0
                    inside = lo <= j <= hi
                    want = (1.0 / (n + math.exp(sink[h]))) if inside else 0.0
                    assert abs(out[b, h, i, d] - want) < 1e-15, (b, h, i, d)


def test_p12_sink_probe():
    B, Hq, Hkv, D, L = 1, 3, 1, 2, 11
    q = np.random.default_rng(12).standard_normal((B, Hq, L, D))
    k = np.zeros((B, Hkv, L, D))
    v = np.ones((B, Hkv, L, D))
    sink = np.array([-1.0, 0.0, 2.5])
    for W in (-1, 1, 4):
        out = oracle.prefill(q, k, v, scale=1.0, window=W, head_sink=sink)
        for h in range(Hq):
            for i in range(L):
                n = _interval_count(i, L, True, W)
                want = n / (n + math.exp(sink[h]))
                np.testing.assert_allclose(out[0, h, i], want, rtol=0, atol=1e-15)
        if W == 1:
            sig = 1.0 / (1.0 + np.exp(sink))
            np.testing.assert_allclose(out[0, :, :, 0], np.repeat(sig[:, None], L, 1), atol=1e-15)


def test_p13_head_mapping_probe():
    B, Hkv, G, D, L = 2, 4, 3, 2, 7
    Hq = Hkv * G
    q = np.random.default_rng(13).standard_normal((B, Hq, L, D))
    k = np.zeros((B, Hkv, L, D))
    v = np.zeros((B, Hkv, L, D))
    for g in range(Hkv):
        v[:, g] = g + 1
    sink = np.linspace(-1, 1, Hq)
    out = oracle.prefill(q, k, v, scale=1.0, window=3, head_sink=sink)
    for h in range(Hq):
        for i in range(L):
            n = _interval_count(i, L, True, 3)
            want = (h // G + 1) * n / (n + math.exp(sink[h]))
            np.testing.assert_allclose(out[:, h, i], want, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# P-14: softcap
# --------------------------------------------------------------------------
def test_p14_huge_cap_is_no_cap():
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 1, 2, 8, 4), _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 8, 4)
    a = oracle.prefill(q, k, v, scale=1.0, softcap=0.0, window=5)
    b = oracle.prefill(q, k, v, scale=1.0, softcap=1e9, window=5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_p14_two_key_closed_form():
    rng = np.random.default_rng(141)
    for c in (0.5, 2.0, 30.0):
        q = rng.standard_normal((1, 1, 1, 3)) * 3
        k = rng.standard_normal((1, 1, 2, 3)) * 3
        v = rng.standard_normal((1, 1, 2, 3))
        out = oracle.prefill(q, k, v, scale=0.8, causal=False, softcap=c)
        x0 = 0.8 * float(q[0, 0, 0] @ k[0, 0, 0])
        x1 = 0.8 * float(q[0, 0, 0] @ k[0, 0, 1])
        w1 = 1.0 / (1.0 + math.exp(-(c * math.tanh(x1 / c) - c * math.tanh(x0 / c))))
        want = (1 - w1) * v[0, 0, 0] + w1 * v[0, 0, 1]
        np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# hand-worked golden examples
# --------------------------------------------------------------------------
def _num(x):
    if isinstance(x, list):
        return [_num(e) for e in x]
    if isinstance(x, str):
        table = {"ln1": 0.0, "ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4),
                 "2*atanh(ln3/2)": 2 * math.atanh(math.log(3) / 2)}
        return table[x]
    return float(x)


def _golden_cases():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked_golden(case):
    if case["kind"] == "rotary":
        got = oracle.rotary.rotate(np.array(_num(case["x"])), case["positions"],
                                   np.array(_num(case["cos"])), np.array(_num(case["sin"])))
        np.testing.assert_allclose(got, np.array(case["expected"], dtype=np.float64), rtol=0, atol=0)
        return
    a = case["attrs"]
    kw = dict(scale=a["scale"], causal=a["causal"], window=a["window"],
              softcap=a["softcap"], smooth_softmax=a["smooth_softmax"],
              head_sink=None if case["head_sink"] is None else _num(case["head_sink"]))
    if case["kind"] == "prefill":
        got = oracle.prefill(np.array(_num(case["q"])), np.array(_num(case["k"])),
                             np.array(_num(case["v"])), **kw)
    else:
        got = oracle.decode(np.array(_num(case["q"])), np.array(_num(case["k_cache"])),
                            np.array(_num(case["v_cache"])), case["seqlens_k"], **kw)
    np.testing.assert_allclose(got, np.array(case["expected"], dtype=np.float64),
                               rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# argument checks
# --------------------------------------------------------------------------
def test_invalid_attributes_raise():
    z = np.zeros((1, 2, 3, 2))
    with pytest.raises(ValueError):
        oracle.prefill(z, z[:, :1], z[:, :1], scale=1.0, window=0)
    with pytest.raises(ValueError):
        oracle.prefill(z, z[:, :1], z[:, :1], scale=1.0, window=-2)
    with pytest.raises(ValueError):
        oracle.prefill(z, z[:, :1], z[:, :1], scale=1.0, causal=False, window=2)
    with pytest.raises(ValueError):
        oracle.prefill(z, z[:, :1], z[:, :1], scale=1.0, softcap=-1.0)
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((1, 3, 3, 2)), z[:, :2], z[:, :2], scale=1.0)
    with pytest.raises(ValueError):
        oracle.decode(z, z, z, [1], scale=1.0)  # total 2 < curr 3


# --------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of the oracle must fail a pin
# --------------------------------------------------------------------------
def _mutant(old, new):
    src = open(oracle_mod.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new,pin", [
    ("((q_abs - j) < window)", "((q_abs - j) <= window)", "p11"),     # window off by one
    ("(j <= q_abs)", "(j < q_abs)", "p11"),                            # diagonal dropped
    ("ok = (j >= 0) & (j < valid)", "ok = (j >= 0) & (j <= valid)", "p11"),  # nonpad edge
    ("g = h // G", "g = h % Hkv", "p13"),                               # head map order
    ("Z = Z + np.exp(s - m)", "Z = Z - np.exp(s - m)", "p7"),          # sink sign
    ("Z = Z + np.exp(s - m)", "Z = Z + np.exp(s)", "p7"),              # sink not shifted
    ("return cap * np.tanh(x / cap)", "return np.tanh(x) * cap", "p14"),  # cap formula
    ("X = scale * (q[b, h, r] @ kbg.T)", "X = (q[b, h, r] @ kbg.T)", "p7"),  # scale dropped
    ("O[~M.any(axis=1)] = 0.0", "pass", "p8"),                          # empty rows
])
def test_pins_catch_planted_mistakes(monkeypatch, old, new, pin):
    mut = _mutant(old, new)
    fake = types.SimpleNamespace(
        attention=mut.attention, prefill=mut.prefill, decode=mut.decode,
        append_kv=mut.append_kv, sink_logits=mut.sink_logits, allowed=mut.allowed)
    monkeypatch.setattr(sys.modules[__name__], "oracle", fake)
    checks = {
        "p11": lambda: [test_p11_mask_probe(*a) for a in [
            (True, 3, None, 12, 12), (True, -1, None, 12, 12), (True, 5, (12, 7), 9, 12)]],
        "p13": test_p13_head_mapping_probe,
        "p7": test_p7_single_key_sink_closed_form,
        "p14": test_p14_two_key_closed_form,
        "p8": test_p8_fully_masked_rows_are_zero,
    }
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            checks[pin]()
