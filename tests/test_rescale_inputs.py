"""CPU checks of the shaped inputs that the lazy-rescale GPU tests use
(windowed_gqa_kv_amd.inputs.shape_logits): the logits follow the prescribed
levels, and the inputs are sensitive to the rescale itself.

Sensitivity: a tile-by-tile online softmax with the lazy rule (move the
running max only when it rises by more than 8 ln 2 nats), written here in
float64, agrees with the oracle on these inputs; the same recurrence with the
rescale of the output or of the denominator left out (the mistakes a
miscompiled or misplaced branch would make) misses the oracle by far more
than the bf16 tolerance.  So a kernel that passes the GPU tests takes the
branch correctly."""

import math

import numpy as np
import pytest

import oracle
from windowed_gqa_kv_amd.inputs import Workload, bursts, generate, shape_logits, staircase, to_f64

THRESHOLD = 8.0 * math.log(2.0)


def _tiled(x, v, tile, broken=None):
    """Rows of softmax(x) @ v by the lazy online recurrence over key tiles."""
    out = np.zeros((x.shape[0], v.shape[1]))
    for i in range(x.shape[0]):
        m, l, o = -np.inf, 0.0, np.zeros(v.shape[1])
        for k0 in range(0, x.shape[1], tile):
            xs = x[i, k0:k0 + tile]
            mt = xs.max()
            if mt == -np.inf:
                continue
            if mt - m > THRESHOLD:
                alpha = math.exp(m - mt) if m > -np.inf else 0.0
                if broken != "l":
                    l *= alpha
                if broken != "o":
                    o *= alpha
                m = mt
            p = np.exp(xs - m)
            l += p.sum()
            o += p @ v[k0:k0 + tile]
        out[i] = o / l
    return out


@pytest.mark.parametrize("profile", [("stair", 7.5, 64), ("bursts", 6.8, 256, 16)])
def test_shaped_logits_follow_levels_and_catch_a_broken_rescale(profile):
    w = Workload("shape", "prefill", "bf16", B=1, Hq=2, Hkv=1, D=128, Lq=64, Lk=1024, causal=False,
                 seed=3)
    lv = staircase(1024, *profile[1:]) if profile[0] == "stair" else bursts(1024, *profile[1:])
    d = shape_logits(w, generate(w), lv, seed=9)
    q, k, v = to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"])
    x = w.sm_scale * (q[0, 0] @ k[0, 0].T)
    # the noise of a query's own component grows with the level's key coefficient
    assert (np.abs(x - lv[None, :]) < 1.5 + 0.03 * lv[None, :]).all()
    want = oracle.prefill(q, k, v, scale=w.sm_scale, causal=False)[0, 0]
    good = _tiled(x, v[0, 0], 64)
    assert np.abs(good - want).max() < 1e-9
    for broken in ("o", "l"):
        bad = _tiled(x, v[0, 0], 64, broken)
        assert np.abs(bad - want).max() > 0.1, broken
