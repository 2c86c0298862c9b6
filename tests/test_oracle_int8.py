"""Pins of the oracle's INT8 KV cache with per-KV-head scales (oracle.int8).

Quantization is checked against values worked out by hand (ties to even,
saturation, NaN, the per-head scale), against torch's round-half-to-even
(a library routine other than the one the oracle uses), by a round trip over
every code, and the quantized decode against the plain decode when every
cached value is exactly a code times its head's scale (the scales then fold
out exactly).  Planted mistakes must fail a pin.
"""

import numpy as np
import pytest
import torch

import oracle

i8 = oracle.int8


def _x(vals, scale=1.0):
    """A [1, 1, 1, n] array of the given multiples of `scale`."""
    return (np.asarray(vals, dtype=np.float64) * scale).reshape(1, 1, 1, -1)


def test_hand_values():
    s = [0.5]
    got = i8.quantize(_x([0.25, 0.75, 1.25, -1.25, 0.74, 63.2, 63.75, 70.0, -70.0], 1.0), s).ravel()
    # x / 0.5: 0.5 -> 0 (tie, even), 1.5 -> 2, 2.5 -> 2, -2.5 -> -2, 1.48 -> 1,
    # 126.4 -> 126, 127.5 -> 127 (clamped), 140 -> 127, -140 -> -127
    assert got.tolist() == [0, 2, 2, -2, 1, 126, 127, 127, -127]
    assert i8.quantize(_x([np.nan, np.inf, -np.inf, 0.0, -0.0]), [1.0]).ravel().tolist() == [0, 127, -127, 0, 0]


def test_matches_torch_round_half_even():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 3, 50, 16)).astype(np.float32) * 40
    sc = np.array([0.37, 1.0, 0.05], dtype=np.float32)
    t = torch.from_numpy(x) * (1.0 / torch.from_numpy(sc)).view(1, 3, 1, 1)  # fp32 reciprocal, fp32 product
    want = torch.clamp(torch.round(t), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(i8.quantize(x, sc), want)


def test_round_trip_every_code():
    codes = np.arange(-127, 128, dtype=np.int8).reshape(1, 1, 1, -1)
    for s in (1.0, 0.25, 2.0 ** -7, 8.0):
        assert np.array_equal(i8.quantize(i8.dequantize(codes, [s]), [s]), codes)


def test_per_head_scales():
    x = np.full((1, 2, 1, 4), 3.0)
    got = i8.quantize(x, [1.0, 0.5])
    assert got[0, 0].ravel().tolist() == [3] * 4 and got[0, 1].ravel().tolist() == [6] * 4
    np.testing.assert_array_equal(i8.dequantize(got, [1.0, 0.5]), x)


def test_quantized_decode_equals_plain_on_representable_caches():
    """Caches whose values are codes times their head's power-of-two scale:
    the INT8 decode equals the plain decode of those values exactly."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, cap, D, curr = 2, 4, 2, 40, 16, 2
    ks, vs = np.array([0.125, 0.25]), np.array([0.5, 0.0625])
    kc = rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, cap, D)).astype(np.int8)
    kn = i8.dequantize(rng.integers(-127, 128, (B, Hkv, curr, D)).astype(np.int8), ks)
    vn = i8.dequantize(rng.integers(-127, 128, (B, Hkv, curr, D)).astype(np.int8), vs)
    q = rng.standard_normal((B, Hq, curr, D))
    s = np.array([30, 12])
    kq, vq = i8.append(kc, vc, kn, vn, s, ks, vs)
    got = i8.decode(q, kq, vq, s, k_scales=ks, v_scales=vs, scale=0.25, window=20)
    kp, vp = oracle.append_kv(i8.dequantize(kc, ks), i8.dequantize(vc, vs), kn, vn, s)
    want = oracle.decode(q, kp, vp, s, scale=0.25, window=20)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("mistake", ["ties_away", "no_clamp", "multiply_scale", "head0_scale", "nan_to_max"])
def test_planted_mistakes_fail_a_pin(mistake):
    def bad(x, scales):
        x = np.asarray(x, dtype=np.float32)
        s = np.asarray(scales, dtype=np.float32)
        if mistake == "head0_scale":
            s = np.full_like(s, s[0])
        r = np.float32(1.0) / s[None, :, None, None]
        t = x * (s[None, :, None, None] if mistake == "multiply_scale" else r)
        t = np.where(np.isnan(t), 127.0 if mistake == "nan_to_max" else 0.0, t)
        q = np.sign(t) * np.floor(np.abs(t) + 0.5) if mistake == "ties_away" else np.rint(t)
        if mistake != "no_clamp":
            q = np.clip(q, -127, 127)
        return np.clip(q, -128, 127).astype(np.int8)
    failed = 0
    for pin in (test_hand_values, test_per_head_scales, test_round_trip_every_code):
        saved = i8.quantize
        try:
            i8.quantize = bad
            pin()
        except AssertionError:
            failed += 1
        finally:
            i8.quantize = saved
    assert failed >= 1, f"no pin caught {mistake}"
