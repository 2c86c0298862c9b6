"""The library's measurement aids (include/gqa_probe.h), which bench.py uses
for context next to its roofline fractions: they launch, return their
status codes, and reject bad arguments on the host."""

import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_mfma_peak_probe_stamps(gpu):
    blocks, iters = 8, 50
    stamps = torch.zeros(blocks * 4 * 4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks * 4, device="cuda")
    assert gpu.gqa_probe_mfma_peak(blocks, iters, _p(stamps), _p(sink), _stream()) == 0
    torch.cuda.synchronize()
    st = stamps.view(-1, 4).cpu().numpy()
    assert (st[:, 1] > st[:, 0]).all() and (st[:, 3] > st[:, 2]).all()
    assert gpu.gqa_probe_mfma_peak(0, iters, _p(stamps), _p(sink), _stream()) == 1


def test_kv_stream_probe_runs_and_checks_arguments(gpu):
    kv_bytes = 1 << 20
    k = torch.ones(kv_bytes, dtype=torch.uint8, device="cuda")
    v = torch.ones(kv_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, device="cuda")
    # in-range units, plus offsets outside the buffers (the kernel reads unit 0 for them)
    offs = [4096 * i for i in range(200)] + [kv_bytes - 8192, kv_bytes - 4096, -4096, kv_bytes, kv_bytes - 16,
                                             1 << 40]
    off = torch.tensor(np.array(offs, dtype=np.int64), device="cuda")
    U = len(offs)
    for rb in (256, 512):
        for grid in (1, 3, 64, 512):
            assert gpu.gqa_probe_kv_stream(grid, rb, _p(k), _p(v), kv_bytes, _p(off), U, _p(sink), _stream()) == 0
    torch.cuda.synchronize()
    assert sink.item() == 0.0
    # no units: nothing streamed
    assert gpu.gqa_probe_kv_stream(4, 256, _p(k), _p(v), kv_bytes, _p(off), 0, _p(sink), _stream()) == 0
    torch.cuda.synchronize()
    # host-side rejections: no launch
    bad = [
        (0, 256, _p(k), _p(v), kv_bytes, _p(off), U),     # no workgroups
        (1, 384, _p(k), _p(v), kv_bytes, _p(off), U),     # a row size the probe does not take
        (1, 256, _p(k), _p(v), 4095, _p(off), U),         # a buffer smaller than one unit
        (1, 512, _p(k), _p(v), 8191, _p(off), U),
        (1, 256, None, _p(v), kv_bytes, _p(off), U),      # a NULL buffer
        (1, 256, _p(k), _p(v), kv_bytes, None, U),        # no offsets for the units
        (1, 256, _p(k), _p(v), kv_bytes, _p(off), 257),   # more than 256 units per workgroup
        (4, 256, _p(k), _p(v), kv_bytes, _p(off), -1),    # a negative count
    ]
    for grid, rb, kp, vp, nb, op, units in bad:
        assert gpu.gqa_probe_kv_stream(grid, rb, kp, vp, nb, op, units, _p(sink), _stream()) == 1
