"""Pins of the oracle's rotary position embedding (oracle.rotary).

Each test checks it against something it does not compute by itself: the
turn of a complex number (numpy's complex product), the hand-worked example
in tests/golden/ (run by test_oracle_pins), invariants of a rotation (lengths
kept, scores depend on the position difference only), and the page's
position rule (a generated token at position seqlens_k; decode rows equal
the tail of the prompt they extend).  Mutation tests at the end plant
plausible mistakes in a copy of the module and check that a pin catches each.
"""

import sys
import types

import numpy as np
import pytest

import oracle
from oracle import rotary as rot_mod
from windowed_gqa_kv_amd.inputs import rotary_tables

rot = oracle.rotary


def _tables(max_pos, D, seed=0):
    """Random angles: a turn per (position, pair), any angle allowed."""
    ang = np.random.default_rng(seed).uniform(-np.pi, np.pi, size=(max_pos, D // 2))
    return np.cos(ang), np.sin(ang), ang


def test_rotate_is_a_complex_turn():
    """(a, b) -> (a + ib) e^{i theta} for the pair (x_i, x_{i+D/2})."""
    rng = np.random.default_rng(1)
    D, L = 16, 9
    x = rng.standard_normal((2, 3, L, D))
    cos, sin, ang = _tables(20, D)
    pos = rng.integers(0, 20, size=(2, 1, L))
    got = rot.rotate(x, pos, cos, sin)
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * ang[np.broadcast_to(pos, x.shape[:-1])])
    np.testing.assert_allclose(got[..., : D // 2], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[..., D // 2:], z.imag, rtol=0, atol=1e-14)


def test_rotate_keeps_pair_lengths_and_undoes_with_negative_angle():
    rng = np.random.default_rng(2)
    D = 8
    x = rng.standard_normal((5, D))
    cos, sin, _ = _tables(7, D, seed=3)
    pos = np.array([0, 3, 6, 2, 2])
    y = rot.rotate(x, pos, cos, sin)
    h = D // 2
    np.testing.assert_allclose(y[:, :h] ** 2 + y[:, h:] ** 2, x[:, :h] ** 2 + x[:, h:] ** 2, rtol=1e-13)
    back = rot.rotate(y, pos, cos, -sin)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-14)


def test_scores_depend_on_position_difference_only():
    """With the usual frequency tables, <R_p q, R_s k> = <R_{p+d} q, R_{s+d} k>."""
    rng = np.random.default_rng(4)
    D = 32
    ang = np.arange(200)[:, None] * 10000.0 ** (-2.0 * np.arange(D // 2) / D)[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    # the float32 tables the GPU tests use are these, rounded once
    c32, s32 = rotary_tables(200, D)
    np.testing.assert_array_equal(c32.numpy(), cos.astype(np.float32))
    np.testing.assert_array_equal(s32.numpy(), sin.astype(np.float32))
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for p, s, d in [(5, 2, 17), (40, 40, 100), (3, 90, 50)]:
        a = rot.rotate(q, p, cos, sin) @ rot.rotate(k, s, cos, sin)
        b = rot.rotate(q, p + d, cos, sin) @ rot.rotate(k, s + d, cos, sin)
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    # and position 0 of those tables is the identity
    np.testing.assert_array_equal(rot.rotate(q, 0, cos, sin), q)


def test_generated_token_sits_at_seqlens_k():
    """A single generated token is turned at position seqlens_k, and the
    cache slot seqlens_k holds the turned key (K rotated before caching)."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, cap = 3, 4, 2, 8, 12
    seq = np.array([0, 5, 11])
    cos, sin, ang = _tables(cap, D, seed=6)
    q = rng.standard_normal((B, Hq, 1, D))
    kn, vn = rng.standard_normal((B, Hkv, 1, D)), rng.standard_normal((B, Hkv, 1, D))
    kc, vc = np.zeros((B, Hkv, cap, D)), np.zeros((B, Hkv, cap, D))
    q_rot, kc2, vc2 = rot.append_kv_rotary(kc, vc, q, kn, vn, seq, cos, sin)

    def turn(x, p):
        z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * ang[p])
        return np.concatenate([z.real, z.imag], axis=-1)

    for b in range(B):
        s = int(seq[b])
        np.testing.assert_allclose(q_rot[b, :, 0], turn(q[b, :, 0], s), atol=1e-14)
        np.testing.assert_allclose(kc2[b, :, s], turn(kn[b, :, 0], s), atol=1e-14)
        np.testing.assert_array_equal(vc2[b, :, s], vn[b, :, 0])
        other = np.ones(cap, bool)
        other[s] = False
        assert not kc2[b, :, other].any() and not vc2[b, :, other].any()


def test_prompt_positions_are_zero_to_s():
    rng = np.random.default_rng(7)
    D, S = 8, 6
    cos, sin, ang = _tables(S, D, seed=8)
    q, k = rng.standard_normal((1, 2, S, D)), rng.standard_normal((1, 1, S, D))
    qr, kr = rot.rotate_prefill(q, k, cos, sin)
    for i in range(S):
        z = (q[0, 1, i, :4] + 1j * q[0, 1, i, 4:]) * np.exp(1j * ang[i])
        np.testing.assert_allclose(qr[0, 1, i], np.concatenate([z.real, z.imag]), atol=1e-14)
        z = (k[0, 0, i, :4] + 1j * k[0, 0, i, 4:]) * np.exp(1j * ang[i])
        np.testing.assert_allclose(kr[0, 0, i], np.concatenate([z.real, z.imag]), atol=1e-14)


@pytest.mark.parametrize("curr,window", [(1, -1), (3, 4), (2, 1)])
def test_rotary_decode_equals_prompt_tail(curr, window):
    """Decoding the last curr tokens (keys turned as they were appended)
    gives the last curr rows of the prompt over the whole sequence."""
    rng = np.random.default_rng(10 + curr)
    B, Hq, Hkv, D, total = 2, 4, 2, 8, 9
    cos, sin, _ = _tables(total, D, seed=11)
    q = rng.standard_normal((B, Hq, total, D))
    k = rng.standard_normal((B, Hkv, total, D))
    v = rng.standard_normal((B, Hkv, total, D))
    qr, kr = rot.rotate_prefill(q, k, cos, sin)
    want = oracle.prefill(qr, kr, v, scale=0.5, window=window)[:, :, total - curr:]
    # the past was cached turned; the step turns its new rows itself
    seq = np.full(B, total - 1)
    past_k = kr.copy()
    past_k[:, :, total - curr:] = 7.0  # slots the step overwrites
    q_rot, kc, vc = rot.append_kv_rotary(past_k, v, q[:, :, total - curr:], k[:, :, total - curr:],
                                         v[:, :, total - curr:], seq, cos, sin)
    got = oracle.decode(q_rot, kc, vc, seq, scale=0.5, window=window)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_prompt_rows_keep_their_positions():
    """Bottom-right prompt (Lq < Lk): its rows are the last Lq rows of the
    full prompt, turned at the same positions."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, Lk, Lq = 1, 2, 1, 8, 10, 4
    cos, sin, _ = _tables(Lk, D, seed=13)
    q = rng.standard_normal((B, Hq, Lk, D))
    k = rng.standard_normal((B, Hkv, Lk, D))
    v = rng.standard_normal((B, Hkv, Lk, D))
    qr, kr = rot.rotate_prefill(q, k, cos, sin)
    want = oracle.prefill(qr, kr, v, scale=0.5, window=3)[:, :, Lk - Lq:]
    qr2, kr2 = rot.rotate_prefill(q[:, :, Lk - Lq:], k, cos, sin)
    got = oracle.prefill(qr2, kr2, v, scale=0.5, window=3)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_rotary_rejects_bad_input():
    cos, sin, _ = _tables(4, 4)
    with pytest.raises(ValueError):
        rot.rotate(np.zeros((2, 4)), [0, 4], cos, sin)  # position past the tables
    with pytest.raises(ValueError):
        rot.rotate(np.zeros((2, 3)), [0, 1], cos, sin)  # odd head size
    with pytest.raises(ValueError):
        rot.rotate(np.zeros((2, 6)), [0, 1], cos, sin)  # tables of the wrong width


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------
def _mutant(old, new):
    src = open(rot_mod.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle.rotary_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "rotary_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new,pins", [
    ("[a * c - b * s, b * c + a * s]", "[a * c + b * s, b * c - a * s]", "complex"),   # turn the other way
    ("[a * c - b * s, b * c + a * s]", "[a * c - b * s, b * c - a * s]", "complex"),   # one sign wrong
    ("a = x[..., :half]\n    b = x[..., half:]", "a = x[..., 0::2]\n    b = x[..., 1::2]", "complex"),  # interleaved pairs
    ("return total[:, None] - curr + np.arange(curr)[None, :]",
     "return total[:, None] - curr + 1 + np.arange(curr)[None, :]", "seqlens"),     # one position late
    ("return (Lk - Lq) + np.arange(Lq), np.arange(Lk)", "return np.arange(Lq), np.arange(Lk)", "tail"),  # prompt offset
])
def test_rotary_pins_catch_planted_mistakes(monkeypatch, old, new, pins):
    mut = _mutant(old, new)
    monkeypatch.setattr(sys.modules[__name__], "rot", mut)
    checks = {
        "complex": test_rotate_is_a_complex_turn,
        "seqlens": test_generated_token_sits_at_seqlens_k,
        "tail": test_prompt_rows_keep_their_positions,
    }
    with pytest.raises((AssertionError, ValueError, IndexError)):
        checks[pins]()
