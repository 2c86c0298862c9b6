"""Pins of the oracle's FP8 (E4M3) KV cache (oracle.fp8).

The code table is checked against torch's float8_e4m3fn type (a library
routine) and against values worked out by hand from the bit layout; encoding
against torch's round-to-nearest-even cast in range, a round trip over every
finite code, hand-picked ties and the saturation rule; the quantized decode
against the plain decode when every cached value is exactly representable
(the scales then fold out exactly).  Planted mistakes must fail a pin.
"""

import sys
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as fp8_mod

f8 = oracle.fp8


def test_code_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = f8.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    assert np.signbit(got[0x80]) and got[0x80] == 0.0


def test_code_table_hand_values():
    """From the layout s.eeee.mmm, bias 7: 0x38 = 0.0111.000 = 1;
    0x7E = 0.1111.110 = 2^8 * 1.75 = 448; 0x01 = 2^-6 * 1/8 = 2^-9;
    0x08 = 2^-6 (least normal); 0xC4 = -(2^1 * 1.5) = -3; 0x7F NaN."""
    v = f8.e4m3_decode([0x38, 0x7E, 0x01, 0x08, 0xC4, 0x7F])
    assert list(v[:5]) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -3.0]
    assert np.isnan(v[5])


def test_encode_round_trips_every_finite_code():
    c = np.array([x for x in range(256) if x not in (0x7F, 0xFF)])
    np.testing.assert_array_equal(f8.e4m3_encode(f8.e4m3_decode(c)), c)


def test_encode_matches_torch_rounding_in_range():
    rng = np.random.default_rng(1)
    t = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 1e-2,
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    want = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(f8.e4m3_encode(t.astype(np.float64)), want)


def test_encode_ties_and_saturation():
    # between 1 (0x38) and 1.125 (0x39): the tie goes to the even code 0x38;
    # between 1.125 (0x39) and 1.25 (0x3A): to 0x3A
    assert list(f8.e4m3_encode([1.0625, 1.1875, -1.0625])) == [0x38, 0x3A, 0xB8]
    # subnormal tie: 2^-10 lies halfway between 0 and 2^-9 -> 0 (even)
    assert list(f8.e4m3_encode([2.0 ** -10, 3 * 2.0 ** -10])) == [0x00, 0x02]
    # beyond the largest finite value: saturate
    assert list(f8.e4m3_encode([449.0, 1e9, -500.0, np.inf])) == [0x7E, 0x7E, 0xFE, 0x7E]
    assert f8.e4m3_encode([np.nan])[0] == 0x7F
    assert f8.e4m3_encode([-1e-30])[0] == 0x80


def test_quantize_uses_the_fp32_reciprocal():
    x = np.array([3.0, -0.7, 100.0], dtype=np.float32)
    r = np.float32(1) / np.float32(0.37)
    np.testing.assert_array_equal(f8.quantize(x, 0.37),
                                  f8.e4m3_encode((x * r).astype(np.float64)))


def test_fp8_decode_equals_plain_decode_on_representable_values():
    """Caches whose values are codes times the scales: quantization is
    lossless and the scales fold out exactly."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, D, cap, curr = 2, 4, 2, 8, 20, 2
    ks, vs = 0.125, 0.5
    kc = f8.e4m3_encode(rng.standard_normal((B, Hkv, cap, D)) * 4)
    vc = f8.e4m3_encode(rng.standard_normal((B, Hkv, cap, D)) * 4)
    kn = f8.e4m3_decode(f8.e4m3_encode(rng.standard_normal((B, Hkv, curr, D)) * 4)) * ks
    vn = f8.e4m3_decode(f8.e4m3_encode(rng.standard_normal((B, Hkv, curr, D)) * 4)) * vs
    q = rng.standard_normal((B, Hq, curr, D))
    seq = np.array([cap - 1, 9])
    kc2, vc2 = f8.append(kc, vc, kn, vn, seq, ks, vs)
    got = f8.decode(q, kc2, vc2, seq, k_scale=ks, v_scale=vs, scale=0.3, window=6)
    kl, vl = oracle.append_kv(f8.e4m3_decode(kc) * ks, f8.e4m3_decode(vc) * vs, kn, vn, seq)
    want = oracle.decode(q, kl, vl, seq, scale=0.3, window=6)
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------
def _mutant(old, new):
    src = open(fp8_mod.__file__).read()
    assert old in src, old
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("2.0 ** (e - 7)", "2.0 ** (e - 8)"),                                       # bias 8
    ("(hi % 2 == 0)", "(hi % 2 == 1)"),                                          # ties to odd
    ("return np.where(np.isnan(t), np.uint8(0x7F), code)",
     "return np.where(np.isnan(t) | (np.abs(t) > E4M3_MAX), np.uint8(0x7F), code)"),  # overflow to NaN
    ("t = np.asarray(x, dtype=np.float32) * r", "t = np.asarray(x, dtype=np.float32) / r"),  # scale inverted
    ("2.0 ** -6 * (m / 8.0)", "2.0 ** -7 * (m / 8.0)"),                          # subnormal exponent
])
def test_fp8_pins_catch_planted_mistakes(monkeypatch, old, new):
    mut = _mutant(old, new)
    monkeypatch.setattr(sys.modules[__name__], "f8", mut)
    caught = False
    try:
        with np.errstate(all="ignore"):
            test_code_table_matches_torch_float8_e4m3fn()
            test_code_table_hand_values()
            test_encode_round_trips_every_finite_code()
            test_encode_matches_torch_rounding_in_range()
            test_encode_ties_and_saturation()
            test_quantize_uses_the_fp32_reciprocal()
            test_fp8_decode_equals_plain_decode_on_representable_values()
    except (AssertionError, ValueError, IndexError):
        caught = True
    assert caught, "no pin caught the planted mistake"
