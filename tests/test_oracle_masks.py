"""Pins of the oracle's caller masks (boolean and additive, broadcast over
[B, Hq, Lq, Lk]; oracle.materialized step 7).

Each test checks the masked oracle against something it does not compute by
itself: torch's scaled_dot_product_attention in float64 (whose boolean mask
has the same True-attends convention and whose float mask is added to the
scaled logits), closed forms with softcap and a sink, invariants (a constant
bias per row changes nothing without a sink; a boolean mask equals the
additive mask of 0 and -inf; broadcast equals repetition) and a hand-worked
example.  Planted mistakes in a copy of the oracle must fail them.
"""

import math
import sys
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import materialized as oracle_mod

mo = oracle


def _case(seed, B=2, Hq=4, Hkv=2, Lq=7, Lk=9, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    v = rng.standard_normal((B, Hkv, Lk, D))
    return rng, q, k, v


def _sdpa(q, k, v, scale, attn_mask):
    G = q.shape[1] // k.shape[1]
    kk = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kk, vv, attn_mask=torch.from_numpy(attn_mask), scale=scale).numpy()


def _band(Lq, Lk, window):
    i = (Lk - Lq) + np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    ok = j <= i
    if window != -1:
        ok &= (i - j) < window
    return ok


@pytest.mark.parametrize("window", [-1, 4])
def test_boolean_mask_matches_library_sdpa(window):
    rng, q, k, v = _case(1)
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    m = rng.random((B, 1, Lq, Lk)) < 0.6
    band = _band(Lq, Lk, window)
    for i in range(Lq):  # every row keeps its earliest key inside the band
        p = Lk - Lq + i
        m[:, :, i, 0 if window == -1 else max(0, p - window + 1)] = True
    full = np.broadcast_to(m & band, (B, Hq, Lq, Lk))
    keep = full.any(-1)
    got = mo.prefill(q, k, v, scale=0.3, window=window, mask=m)
    want = _sdpa(q, k, v, 0.3, np.ascontiguousarray(full))
    np.testing.assert_allclose(got[keep], want[keep], rtol=0, atol=1e-12)


def test_additive_mask_matches_library_sdpa():
    rng, q, k, v = _case(2)
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    bias = rng.standard_normal((1, Hq, Lq, Lk)) * 2.0
    band = _band(Lq, Lk, -1)
    got = mo.prefill(q, k, v, scale=0.5, mask=bias)
    want = _sdpa(q, k, v, 0.5, np.ascontiguousarray(
        np.broadcast_to(np.where(band, bias, -np.inf), (B, Hq, Lq, Lk))))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_boolean_mask_is_the_additive_mask_of_zero_and_minus_inf():
    rng, q, k, v = _case(3)
    m = rng.random((2, 4, 7, 9)) < 0.5
    sink = np.random.default_rng(30).standard_normal(4)
    a = mo.prefill(q, k, v, scale=0.4, softcap=3.0, head_sink=sink, mask=m)
    b = mo.prefill(q, k, v, scale=0.4, softcap=3.0, head_sink=sink, mask=np.where(m, 0.0, -np.inf))
    np.testing.assert_array_equal(a, b)
    # and an all-True mask is no mask at all
    np.testing.assert_array_equal(mo.prefill(q, k, v, scale=0.4, mask=np.ones((1, 1, 7, 9), bool)),
                                  mo.prefill(q, k, v, scale=0.4))


def test_constant_bias_per_row_changes_nothing_without_a_sink():
    rng, q, k, v = _case(4)
    c = rng.standard_normal((2, 4, 7, 1)) * 5
    a = mo.prefill(q, k, v, scale=0.4, window=5, mask=np.broadcast_to(c, (2, 4, 7, 9)))
    b = mo.prefill(q, k, v, scale=0.4, window=5)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_bias_enters_before_softcap_and_not_the_sink():
    """One allowed key: O = logistic(c tanh((x + beta)/c) - s) * v."""
    x_q, x_k, beta, c, s = 1.3, 0.7, -0.4, 2.0, 0.25
    q = np.array([[[[x_q]]]])
    k = np.array([[[[x_k]]]])
    v = np.array([[[[3.0]]]])
    got = mo.prefill(q, k, v, scale=1.0, softcap=c, head_sink=[s], mask=np.array([[[[beta]]]]))
    z = c * math.tanh((x_q * x_k + beta) / c)
    want = 3.0 / (1.0 + math.exp(s - z))
    assert abs(float(got[0, 0, 0, 0]) - want) < 1e-14


def test_rows_whose_keys_are_all_masked_are_zero():
    rng, q, k, v = _case(5)
    m = np.ones((2, 4, 7, 9), bool)
    m[1, 2, 3] = False
    bias = np.zeros((2, 4, 7, 9))
    bias[0, 1, 4] = -np.inf
    for mask in (m, bias):
        out = mo.prefill(q, k, v, scale=0.4, smooth_softmax=True, mask=mask)
        assert np.isfinite(out).all()
    assert not mo.prefill(q, k, v, scale=0.4, smooth_softmax=True, mask=m)[1, 2, 3].any()
    assert not mo.prefill(q, k, v, scale=0.4, smooth_softmax=True, mask=bias)[0, 1, 4].any()
    # a -inf bias removes the key even under softcap (tanh would turn it finite)
    capped = mo.prefill(q, k, v, scale=0.4, softcap=2.0, mask=bias)
    assert np.isfinite(capped).all() and not capped[0, 1, 4].any()
    one = bias.copy()
    one[0, 1, 4, 0] = 0.0  # a single key left: its value row, exactly
    np.testing.assert_allclose(mo.prefill(q, k, v, scale=0.4, softcap=2.0, mask=one)[0, 1, 4],
                               v[0, 0, 0], rtol=0, atol=1e-14)


def test_broadcast_mask_equals_its_repetition_and_decode_masks_cache_slots():
    rng, q, k, v = _case(6)
    m = rng.random((1, 1, 7, 9)) < 0.7
    a = mo.prefill(q, k, v, scale=0.4, mask=m)
    b = mo.prefill(q, k, v, scale=0.4, mask=np.repeat(np.repeat(m, 2, 0), 4, 1))
    np.testing.assert_array_equal(a, b)
    # decode: the mask's key axis is the cache slot; masking slot j equals
    # removing key j by a boolean mask over the same slots of the prompt tail
    seq = np.array([8, 8])
    dm = rng.random((2, 4, 3, 9)) < 0.6
    dm[..., 8] = True
    got = mo.decode(q[:, :, :3], k, v, seq, scale=0.4, mask=dm)
    full = np.ones((2, 4, 9, 9), bool)
    full[:, :, 6:] = dm
    want = mo.prefill(np.concatenate([np.zeros_like(q[:, :, :6]), q[:, :, :3]], axis=2)[:, :, :9],
                      k, v, scale=0.4, mask=full)[:, :, 6:]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_hand_worked_bias_example():
    """One query, two keys with logit 0, bias (0, ln 3): weights 1 and 3,
    O = (4 + 3 * 8) / 4 = 7 (worked on paper)."""
    q = np.array([[[[0.0]]]])
    k = np.array([[[[1.0], [1.0]]]])
    v = np.array([[[[4.0], [8.0]]]])
    out = mo.prefill(q, k, v, scale=1.0, causal=False, mask=np.array([[[[0.0, math.log(3.0)]]]]))
    assert abs(float(out[0, 0, 0, 0]) - 7.0) < 1e-14
    # the boolean mask keeping only key 1: O = 8
    out = mo.prefill(q, k, v, scale=1.0, causal=False, mask=np.array([[[[False, True]]]]))
    assert float(out[0, 0, 0, 0]) == 8.0


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------
def _mutant(old, new):
    src = open(oracle_mod.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle_mask_mutant")
    exec(compile(src.replace(old, new), "oracle_mask_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("X = X + np.where(M, mask[b, h, r], 0.0)", "X = X - np.where(M, mask[b, h, r], 0.0)"),   # bias sign
    ("X = X + np.where(M, mask[b, h, r], 0.0)\n                    X = softcap_fn(X, softcap)",
     "X = softcap_fn(X, softcap)\n                    X = X + np.where(M, mask[b, h, r], 0.0)"),  # bias after cap
    ("M = M & mask[b, h, r]", "M = M"),                                                        # bool mask ignored
    ("M = M & (mask[b, h, r] > -np.inf)", "M = M"),                                           # -inf not excluded
    ("mask = np.broadcast_to(mask, (B, Hq, Lq, Lk))",
     "mask = np.broadcast_to(mask, (B, Hq, Lq, Lk))[:, ::-1]"),                               # wrong head
])
def test_mask_pins_catch_planted_mistakes(monkeypatch, old, new):
    mut = _mutant(old, new)
    fake = types.SimpleNamespace(prefill=mut.prefill, decode=mut.decode)
    monkeypatch.setattr(sys.modules[__name__], "mo", fake)
    caught = False
    try:
        with np.errstate(all="ignore"):
            test_boolean_mask_matches_library_sdpa(-1)
            test_additive_mask_matches_library_sdpa()
            test_bias_enters_before_softcap_and_not_the_sink()
            test_rows_whose_keys_are_all_masked_are_zero()
            test_hand_worked_bias_example()
    except (AssertionError, ValueError, RuntimeError):
        caught = True
    assert caught, "no pin caught the planted mistake"
