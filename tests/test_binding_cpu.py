"""The torch binding rejects malformed tensors before any pointer reaches the
library: shapes against the plan, the dtypes and lengths of the per-batch and
per-head arrays, and tensors that are not on the GPU of q.  Runs on the CPU
(every call here fails in the binding, so no device is touched)."""

import pytest
import torch

from windowed_gqa_kv_amd import binding as bd

H, HKV, D = 8, 2, 64


def plan(**kw):
    base = dict(dtype="bf16", max_batch=4, max_q_len=16, max_kv_len=256)
    base.update(kw)
    return bd.Plan(H, HKV, D, **base)


def z(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_prefill_rejections():
    p = plan()
    q, k = z(2, H, 16, D), z(2, HKV, 32, D)
    with pytest.raises(ValueError, match="expected"):
        p.prefill(z(2, H, 16, 32), k, k)                       # head size
    with pytest.raises(ValueError, match="expected"):
        p.prefill(q, z(2, 3, 32, D), z(2, 3, 32, D))            # KV head count
    with pytest.raises(ValueError, match="differ"):
        p.prefill(q, k, z(2, HKV, 33, D))
    with pytest.raises(ValueError, match="batches"):
        p.prefill(q, z(3, HKV, 32, D), z(3, HKV, 32, D))
    with pytest.raises(TypeError, match="int64"):
        p.prefill(q, k, k, nonpad_kv_seqlen=torch.tensor([1, 2], dtype=torch.int32))
    with pytest.raises(ValueError, match="at least 2"):
        p.prefill(q, k, k, nonpad_kv_seqlen=torch.tensor([1], dtype=torch.int64))
    with pytest.raises(TypeError, match="float32"):
        p.prefill(q, k, k, head_sink=torch.zeros(H, dtype=torch.float64))
    with pytest.raises(ValueError, match="at least 8"):
        p.prefill(q, k, k, head_sink=torch.zeros(H - 1))
    with pytest.raises(TypeError, match="dtype"):
        p.prefill(q.float(), k, k)
    with pytest.raises(ValueError, match="on a GPU"):
        p.prefill(q, k, k)                                       # well-formed, but host memory


def test_decode_and_append_rejections():
    p = plan()
    q, kc = z(2, H, 1, D), z(2, HKV, 256, D)
    seq = torch.tensor([10, 20], dtype=torch.int32)
    with pytest.raises(TypeError, match="int32"):
        p.decode(q, kc, kc, seq.long())
    with pytest.raises(ValueError, match="at least 2"):
        p.decode(q, kc, kc, seq[:1])
    with pytest.raises(ValueError, match="required"):
        p.decode(q, kc, kc, None)
    with pytest.raises(ValueError, match="fewer than"):
        p.decode(q, z(1, HKV, 256, D), z(1, HKV, 256, D), seq)
    with pytest.raises(ValueError, match="workspace"):
        p.decode(q, kc, kc, seq, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="on a GPU"):
        p.decode(q, kc, kc, seq, workspace=torch.zeros(p.workspace_size(), dtype=torch.uint8))
    with pytest.raises(ValueError, match="on a GPU"):
        p.decode_noalloc(q, kc, kc, seq)
    with pytest.raises(TypeError, match="float32"):
        p.decode_noalloc(q, kc, kc, seq, head_sink=torch.zeros(H, dtype=torch.float16))
    with pytest.raises(ValueError, match="expected"):
        p.append_kv(z(2, HKV, 1, 32), z(2, HKV, 1, 32), kc, kc, seq)
    with pytest.raises(TypeError, match="int32"):
        p.append_kv(z(2, HKV, 1, D), z(2, HKV, 1, D), kc, kc, seq.float())
    with pytest.raises(ValueError, match="on a GPU"):
        p.append_kv(z(2, HKV, 1, D), z(2, HKV, 1, D), kc, kc, seq)


def test_fp8_and_rotary_rejections():
    p = plan()
    q = z(2, H, 1, D)
    c8 = torch.zeros(2, HKV, 256, D, dtype=torch.uint8)
    seq = torch.tensor([10, 20], dtype=torch.int32)
    with pytest.raises(TypeError, match="uint8"):
        p.decode_fp8(q, z(2, HKV, 256, D), z(2, HKV, 256, D), seq, 1.0, 1.0)
    with pytest.raises(ValueError, match="expected"):
        p.decode_fp8(q, torch.zeros(2, HKV, 256, 32, dtype=torch.uint8), c8, seq, 1.0, 1.0)
    with pytest.raises(ValueError, match="on a GPU"):
        p.decode_fp8(q, c8, c8, seq, 1.0, 1.0, workspace=torch.zeros(p.workspace_size(), dtype=torch.uint8))
    cos = torch.zeros(256, D // 2)
    with pytest.raises(ValueError, match="x must be"):
        p.apply_rotary(z(2, H, 4, 32), 0, cos, cos)
    with pytest.raises(ValueError, match="on a GPU"):
        p.apply_rotary(z(2, H, 4, D), 0, cos, cos)
    with pytest.raises(ValueError, match="differ in batch"):
        p.append_kv_rotary(z(2, H, 2, D), z(2, HKV, 1, D), z(2, HKV, 1, D), c8.bfloat16(), c8.bfloat16(),
                           seq, cos, cos)
