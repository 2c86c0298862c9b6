"""gqa_last_path names the kernel each call ran: the matrix-core prefill and
decode where they apply, the one-wavefront-per-row streaming kernel where
they do not (fp32 plans, an odd head size, more row tiles than one decode
launch takes, a mask layout the matrix cores cannot read)."""

import pytest
import torch

from windowed_gqa_kv_amd import binding as bd

pytestmark = pytest.mark.gpu


def _plan(D, dtype, **kw):
    base = dict(dtype=dtype, max_batch=64, max_q_len=64, max_kv_len=256)
    base.update(kw)
    return bd.Plan(8, 2, D, **base)


@pytest.mark.parametrize("D,dtype,want", [(128, "bf16", bd.GQA_PATH_MATRIX_PREFILL),
                                          (32, "f16", bd.GQA_PATH_MATRIX_PREFILL),
                                          (256, "bf16", bd.GQA_PATH_MATRIX_PREFILL),
                                          (96, "bf16", bd.GQA_PATH_STREAMING),
                                          (64, "f32", bd.GQA_PATH_STREAMING)])
def test_prefill_path(gpu, D, dtype, want):
    p = _plan(D, dtype)
    t = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    q = torch.randn(1, 8, 40, D, device="cuda").to(t)
    k = torch.randn(1, 2, 40, D, device="cuda").to(t)
    p.prefill(q, k, k)
    assert bd.gqa_last_path() == want, bd.PATH_NAMES[bd.gqa_last_path()]
    if D == 128:  # a mask whose rows are not 8-byte aligned goes to the streaming kernel
        m = torch.ones(1, 1, 40, 41, dtype=torch.bool, device="cuda")[..., :40]
        p.prefill(q, k, k, mask=m)
        assert bd.gqa_last_path() == bd.GQA_PATH_STREAMING
        m = torch.ones(1, 1, 40, 40, dtype=torch.bool, device="cuda")
        p.prefill(q, k, k, mask=m)
        assert bd.gqa_last_path() == bd.GQA_PATH_MATRIX_PREFILL
    torch.cuda.synchronize()


def test_decode_path(gpu):
    p = bd.Plan(64, 16, 64, dtype="bf16", max_batch=40, max_q_len=16, max_kv_len=64)
    seq = torch.full((40,), 30, dtype=torch.int32, device="cuda")
    kc = torch.zeros(40, 16, 64, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.randn(32, 64, 16, 64, device="cuda").bfloat16()
    p.decode(q, kc, kc, seq[:32])          # 32 * 16 * 4 = 2048 row tiles
    assert bd.gqa_last_path() == bd.GQA_PATH_MATRIX_DECODE
    q = torch.randn(33, 64, 16, 64, device="cuda").bfloat16()
    p.decode(q, kc, kc, seq[:33])          # 2112 row tiles
    assert bd.gqa_last_path() == bd.GQA_PATH_STREAMING
    p.append_kv(kc[:1, :, :1], kc[:1, :, :1], kc, kc, seq[:1])
    assert bd.gqa_last_path() == bd.GQA_PATH_NONE
    torch.cuda.synchronize()
