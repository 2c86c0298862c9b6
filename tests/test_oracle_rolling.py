"""Pins of the oracle's rolling KV cache (oracle.rolling).

The page's own statement is the pin: attention over the rolling buffer equals
the window applied as a mask over the full cache.  The tests build the full
history directly (never through the ring), fill a ring by a sequence of steps
of varying length that wraps it several times, and compare decodes.  Planted
mistakes in a copy of the module must fail them.
"""

import sys
import types

import numpy as np
import pytest

import oracle
from oracle import rolling as roll_mod

roll = oracle.rolling


def _history(rng, B, Hkv, total, D):
    return rng.standard_normal((B, Hkv, total, D)), rng.standard_normal((B, Hkv, total, D))


def _fill_ring(C, k_hist, v_hist, steps):
    """Append the history to an empty ring in steps of the given lengths."""
    B, Hkv, T, D = k_hist.shape
    kr = np.full((B, Hkv, C, D), 5.0)  # never-written slots hold junk
    vr = np.full((B, Hkv, C, D), -5.0)
    pos = 0
    for n in steps:
        seq = np.full(B, pos + n - 1)
        kr, vr = roll.append(kr, vr, k_hist[:, :, pos:pos + n], v_hist[:, :, pos:pos + n], seq)
        pos += n
    assert pos == T
    return kr, vr


@pytest.mark.parametrize("C,W,curr,steps", [
    (7, 5, 3, [4, 3, 3, 1, 2, 5, 3]),        # C = W + curr - 1 exactly, wrapped three times
    (10, 4, 1, [9, 1, 1, 1, 1, 1, 1, 1]),    # single-token steps across the wrap
    (16, 6, 4, [3, 8, 4, 4, 4, 4, 4, 4, 4]),  # larger ring than needed
    (6, 6, 1, [6, 1]),                        # ring exactly full, then one wrap
])
def test_rolling_decode_equals_window_over_full_history(C, W, curr, steps):
    rng = np.random.default_rng(C * 100 + W * 10 + curr)
    B, Hq, Hkv, D = 2, 4, 2, 8
    total = sum(steps)
    assert steps[-1] == curr
    k_hist, v_hist = _history(rng, B, Hkv, total, D)
    kr, vr = _fill_ring(C, k_hist, v_hist, steps)
    q = rng.standard_normal((B, Hq, curr, D))
    seq = np.full(B, total - 1)
    sink = rng.standard_normal(Hq)
    got = roll.decode(q, kr, vr, seq, scale=0.4, window=W, head_sink=sink)
    want = oracle.decode(q, k_hist, v_hist, seq, scale=0.4, window=W, head_sink=sink)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_append_writes_only_the_step_slots_across_the_wrap():
    rng = np.random.default_rng(3)
    B, Hkv, C, D, curr = 2, 2, 8, 4, 4
    kr = rng.standard_normal((B, Hkv, C, D))
    vr = rng.standard_normal((B, Hkv, C, D))
    kn, vn = rng.standard_normal((B, Hkv, curr, D)), rng.standard_normal((B, Hkv, curr, D))
    seq = np.array([6 + curr - 1, 29 + curr - 1])  # step positions 6..9 and 29..32
    k2, v2 = roll.append(kr, vr, kn, vn, seq)
    for b, slots in enumerate([[6, 7, 0, 1], [5, 6, 7, 0]]):
        for t, s in enumerate(slots):
            np.testing.assert_array_equal(k2[b, :, s], kn[b, :, t])
            np.testing.assert_array_equal(v2[b, :, s], vn[b, :, t])
        rest = [s for s in range(C) if s not in slots]
        np.testing.assert_array_equal(k2[b][:, rest], kr[b][:, rest])
        np.testing.assert_array_equal(v2[b][:, rest], vr[b][:, rest])


def test_overwritten_positions_are_absent_from_the_history():
    C = 5
    ring = np.arange(2 * 1 * C * 1, dtype=np.float64).reshape(2, 1, C, 1)
    hist = roll.linear_history(ring, np.array([11, 3]))  # totals 12 and 4
    assert np.isnan(hist[0, 0, :7]).all()
    assert [hist[0, 0, j, 0] for j in range(7, 12)] == [ring[0, 0, j % C, 0] for j in range(7, 12)]
    assert [hist[1, 0, j, 0] for j in range(4)] == [ring[1, 0, j, 0] for j in range(4)]  # not wrapped yet
    assert np.isnan(hist[1, 0, 4:]).all()


def test_batches_of_different_lengths():
    """Per-batch histories of different lengths (some never wrapped); the
    ring is filled by placing position p at slot p mod C directly."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, C, W, curr = 3, 4, 2, 8, 9, 7, 3
    totals = np.array([40, 12, 5])
    k_hist, v_hist = _history(rng, B, Hkv, int(totals.max()), D)
    kr = rng.standard_normal((B, Hkv, C, D))
    vr = rng.standard_normal((B, Hkv, C, D))
    for b in range(B):
        for p in range(max(0, totals[b] - C), totals[b]):
            kr[b, :, p % C] = k_hist[b, :, p]
            vr[b, :, p % C] = v_hist[b, :, p]
    q = rng.standard_normal((B, Hq, curr, D))
    got = roll.decode(q, kr, vr, totals - 1, scale=0.5, window=W, smooth_softmax=True)
    want = oracle.decode(q, k_hist, v_hist, totals - 1, scale=0.5, window=W, smooth_softmax=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_far_positions_give_the_same_result():
    """Moving every position by a multiple of the ring (same slots) leaves
    the decode unchanged: only position differences matter."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, C, W, curr = 2, 4, 2, 8, 9, 6, 4
    ring_k, ring_v = rng.standard_normal((B, Hkv, C, D)), rng.standard_normal((B, Hkv, C, D))
    q = rng.standard_normal((B, Hq, curr, D))
    near = np.array([20, 13])
    far = near + 1000 * C
    a = roll.decode(q, ring_k, ring_v, near, scale=0.3, window=W)
    b = roll.decode(q, ring_k, ring_v, far, scale=0.3, window=W)
    np.testing.assert_array_equal(a, b)


def test_rolling_rejects_a_ring_that_loses_needed_keys():
    z = np.zeros((1, 2, 1, 4))
    ring = np.zeros((1, 1, 6, 4))
    with pytest.raises(ValueError):
        roll.decode(np.zeros((1, 2, 3, 4)), ring, ring, [20], scale=1.0, window=5)  # 6 < 5 + 3 - 1
    with pytest.raises(ValueError):
        roll.decode(z, ring, ring, [20], scale=1.0, window=-1)  # no window
    roll.decode(np.zeros((1, 2, 2, 4)), ring, ring, [20], scale=1.0, window=5)  # 6 >= 5 + 2 - 1


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------
def _mutant(old, new):
    src = open(roll_mod.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle.rolling_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "rolling_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("return np.asarray(p) % capacity", "return (np.asarray(p) + 1) % capacity"),          # slot shifted
    ("s = int(slot_of(total[b] - curr + t, C))", "s = int(slot_of(total[b] - curr + t - 1, C))"),  # append late
    ("range(max(start, int(total[b]) - C), int(total[b]))",
     "range(max(start, int(total[b]) - C + 1), int(total[b]))"),                           # oldest kept key dropped
    ("start = int(max(0, total.min() - C))", "start = int(max(0, total.max() - C))"),     # trims keys a batch needs
    ("if C < window + curr - 1:", "if C < window:"),                                        # capacity rule too weak
])
def test_rolling_pins_catch_planted_mistakes(monkeypatch, old, new):
    mut = _mutant(old, new)
    monkeypatch.setattr(sys.modules[__name__], "roll", mut)
    caught = False
    try:
        for args in [(7, 5, 3, [4, 3, 3, 1, 2, 5, 3]), (10, 4, 1, [9, 1, 1, 1, 1, 1, 1, 1])]:
            test_rolling_decode_equals_window_over_full_history(*args)
        test_rolling_decode_equals_window_over_full_history(16, 6, 4, [3, 8, 4, 4, 4, 4, 4, 4, 4])
        test_append_writes_only_the_step_slots_across_the_wrap()
        test_batches_of_different_lengths()
        test_overwritten_positions_are_absent_from_the_history()
        test_rolling_rejects_a_ring_that_loses_needed_keys()
    except (AssertionError, ValueError, pytest.fail.Exception):
        caught = True
    assert caught, "no pin caught the planted mistake"
