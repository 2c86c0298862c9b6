"""Decode on caches whose positions are about 2^24 elements apart (positions
outermost, the KV heads of a position adjacent), on 16-bit and FP8 caches,
against the oracle.  The matrix-core decode loads a unit of 16 consecutive
rows from one base address plus per-lane 32-bit offsets only when the row
strides are below 2^24 elements; at 2^24 + 256 it takes per-lane 64-bit row
addresses.  Both sides of that line are checked."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare
from windowed_gqa_kv_amd import binding as bd
from windowed_gqa_kv_amd.inputs import to_f64

pytestmark = pytest.mark.gpu

HQ, HKV, D, CAP, VALID = 4, 2, 128, 40, 37


def _strided_cache(row, dtype, rows):
    """A [1, HKV, CAP, D] view over a zeroed buffer: element (0, h, s, d) at
    s * row + h * D + d; positions 0 .. VALID - 1 hold `rows` [HKV, VALID, D]."""
    n = (CAP - 1) * row + HKV * D
    buf = torch.zeros(n, dtype=dtype, device="cuda")
    view = buf.as_strided((1, HKV, CAP, D), (n, D, row, 1))
    for s in range(VALID):
        view[0, :, s, :] = rows[:, s, :].to("cuda")
    return view


@pytest.mark.parametrize("row", [(1 << 24) - 256, (1 << 24) + 256])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_decode_with_huge_row_strides(gpu, row, kind):
    g = torch.Generator().manual_seed(row % 1000 + (kind == "fp8"))
    q = torch.randn(1, HQ, 1, D, generator=g).to(torch.bfloat16)
    k = torch.randn(HKV, VALID, D, generator=g)
    v = torch.randn(HKV, VALID, D, generator=g)
    seq = torch.tensor([VALID - 1], dtype=torch.int32)
    scale = D ** -0.5
    plan = bd.Plan(HQ, HKV, D, dtype="bf16", scale=scale, max_batch=1, max_q_len=1, max_kv_len=CAP)
    if kind == "bf16":
        kr, vr = k.to(torch.bfloat16), v.to(torch.bfloat16)
        kc = _strided_cache(row, torch.bfloat16, kr)
        vc = _strided_cache(row, torch.bfloat16, vr)
        assert kc.stride(2) == row
        out = plan.decode(q.cuda(), kc, vc, seq.cuda())
        torch.cuda.synchronize()
        assert bd.gqa_last_path() == bd.GQA_PATH_MATRIX_DECODE
        want = oracle.materialized.decode(to_f64(q), to_f64(kc), to_f64(vc), seq.numpy().astype(np.int64),
                                          scale=scale)
    else:
        ks, vs = 0.02, 0.03
        kcodes = (k / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        vcodes = (v / vs).to(torch.float8_e4m3fn).view(torch.uint8)
        kc = _strided_cache(row, torch.uint8, kcodes)
        vc = _strided_cache(row, torch.uint8, vcodes)
        out = plan.decode_fp8(q.cuda(), kc, vc, seq.cuda(), ks, vs)
        torch.cuda.synchronize()
        want = oracle.fp8.decode(to_f64(q), kc.cpu().numpy(), vc.cpu().numpy(), seq.numpy().astype(np.int64),
                                 k_scale=ks, v_scale=vs, scale=scale)
    compare(out, want, "bf16", f"{kind} decode, row stride {row}")
