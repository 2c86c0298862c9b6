"""The seeded generator: determinism, shapes, dtypes and the length recipes."""

import numpy as np
import torch

from windowed_gqa_kv_amd.inputs import WORKLOADS, generate, to_f64


def test_generation_is_deterministic_and_rounded():
    w = WORKLOADS[1]
    a, b = generate(w), generate(w)
    for key in ("q", "k", "v", "head_sink"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.float32 and a["q"].shape == (1, 4, 64, 32)
    assert a["k"].shape == (1, 2, 64, 32) and a["head_sink"].shape == (4,)
    c = generate(w, seed=5)
    assert not torch.equal(a["q"], c["q"])


def test_decode_recipe_small_shape():
    w = WORKLOADS[2].with_(Lk=64, seqlens=("uniform", 10, 64))
    d = generate(w)
    assert d["k_cache"].dtype == torch.bfloat16 and d["k_cache"].shape == (8, 8, 64, 128)
    assert d["k_new"].shape == (8, 8, 1, 128)
    s = d["seqlens_k"].numpy()
    assert s.dtype == np.int32 and s.min() >= 10 and s.max() < 64
    # draws come after q, k, v, k_new, v_new in that order
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((8, 32, 1, 128), dtype=np.float32)
    assert np.array_equal(to_f64(d["q"]), torch.from_numpy(q).to(torch.bfloat16).double().numpy())


def test_value_scale_and_bf16_rounding():
    w = WORKLOADS[3].with_(Lq=16, Lk=16, Hq=2, Hkv=1)
    d = generate(w)
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((1, 2, 16, 128), dtype=np.float32) * np.float32(0.5)
    want = torch.from_numpy(q).to(torch.bfloat16)
    assert torch.equal(d["q"], want)
    assert d["nonpad"] is None and d["head_sink"] is None


def test_workload_table():
    assert [WORKLOADS[i].name for i in range(1, 6)] == [
        "tiny_prefill_fp32", "decode_1tok_bf16", "long_prefill_bf16",
        "spec_decode_bf16", "gqa_prefill_large_bf16"]
    assert WORKLOADS[4].sm_scale == 1 / 16
    assert WORKLOADS[5].nonpad == (32768, 24576)
