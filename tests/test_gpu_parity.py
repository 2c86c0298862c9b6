"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs.  Tolerances: max-abs 1e-5 for fp32; max-abs 2e-2 and
mean-abs 2e-3 for bf16/fp16 outputs."""

import zlib

import numpy as np
import pytest
import torch

from gpu_util import (compare, gpu_decode, gpu_prefill, make_plan, oracle_decode,
                      oracle_prefill)
from windowed_gqa_kv_amd.inputs import WORKLOADS, Workload, generate, to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------
# the five reference workloads
# --------------------------------------------------------------------------
def test_workload1_tiny_prefill_fp32(gpu):
    w = WORKLOADS[1]
    d = generate(w)
    got = gpu_prefill(w, d)
    want = oracle_prefill(w, d)
    _say(f"w1 err {compare(got, want, 'f32', 'w1')}")


def test_workload2_single_token_decode(gpu):
    w = WORKLOADS[2]
    d = generate(w)
    out, kc, vc = gpu_decode(w, d)
    want = oracle_decode(w, d)
    _say(f"w2 err {compare(out, want, 'bf16', 'w2')}")
    # the append is a byte copy: compare the written slots bitwise
    s = d["seqlens_k"].numpy()
    for b in range(w.B):
        assert torch.equal(kc[b, :, s[b]].cpu(), d["k_new"][b, :, 0])
        assert torch.equal(vc[b, :, s[b]].cpu(), d["v_new"][b, :, 0])


def _sample_rows(L, extra, seed, n_rand=32):
    rng = np.random.default_rng(seed)
    rows = set(range(0, min(L, 96))) | set(range(max(0, L - 64), L))
    for e in extra:
        rows |= set(r for r in range(e - 3, e + 4) if 0 <= r < L)
    rows |= set(rng.integers(0, L, n_rand).tolist())
    return np.array(sorted(rows))


def test_workload3_long_prefill_sampled(gpu):
    w = WORKLOADS[3]
    d = generate(w)
    got = gpu_prefill(w, d)
    rows = _sample_rows(w.Lq, [w.window - 1, w.window, 4160], seed=3)
    want = oracle_prefill(w, d, rows=rows)
    _say(f"w3 err {compare(got[:, :, rows], want, 'bf16', 'w3')}")


def test_workload4_spec_decode(gpu):
    w = WORKLOADS[4]
    d = generate(w)
    out, _, _ = gpu_decode(w, d)
    want = oracle_decode(w, d)
    _say(f"w4 err {compare(out, want, 'bf16', 'w4')}")


def _w5_rows():
    """The large prefill's sampled rows: rows 0-127, the window edge
    (8190-8194), batch 1's padding edge (24570-24582), the last rows that
    still see batch 1's last key 24575 (up to 24575 + 8191 = 32766), the last
    128 rows (row 32767 of batch 1 sees no key) and 384 seeded random rows --
    about 640 rows for every (batch, head)."""
    rng = np.random.default_rng(55)
    rows = set(range(128)) | set(range(8190, 8195)) | set(range(24570, 24583))
    rows |= set(range(32766 - 40, 32767)) | set(range(32768 - 128, 32768))
    rows |= set(rng.integers(128, 32768 - 128, 384).tolist())
    rows = np.array(sorted(rows))
    assert rows.min() >= 0 and rows.max() < 32768
    return rows


@pytest.fixture(scope="module")
def w5_run(gpu):
    """One run of the large GQA prefill; keeps the sampled rows of every head."""
    w = WORKLOADS[5]
    d = generate(w)
    got = gpu_prefill(w, d)
    rows = _w5_rows()
    assert 0 <= rows.min() and rows.max() < w.Lq  # indexes on the GPU: checked on the host
    sample = got[:, :, torch.from_numpy(rows).cuda()].cpu()
    empty_row_nonzero = torch.count_nonzero(got[1, :, 32767]).item()
    del got
    torch.cuda.empty_cache()
    _say(f"w5: {len(rows)} rows per (batch, head) sampled")
    return w, d, rows, sample, empty_row_nonzero


@pytest.mark.parametrize("h0", range(0, 64, 8))
def test_workload5_large_gqa_prefill_sampled(w5_run, h0):
    """Every (batch, head) of the large prefill on ~640 rows against the
    oracle, eight heads per test (the oracle takes a few seconds per head)."""
    from concurrent.futures import ThreadPoolExecutor
    w, d, rows, sample, empty_row_nonzero = w5_run
    heads = list(range(h0, h0 + 8))
    with ThreadPoolExecutor(4) as ex:
        parts = list(ex.map(lambda h: oracle_prefill(w, d, rows=rows, heads=[h])[h], heads))
    wnt = np.stack(parts, axis=1)
    _say(f"w5 heads {h0}-{h0 + 7} err {compare(sample[:, heads], wnt, 'bf16', f'w5 heads {h0}..')}")
    # batch 1 row 32767 sees no key at all
    assert empty_row_nonzero == 0


# --------------------------------------------------------------------------
# sweeps: tile boundaries, ragged tails, windows, sinks, softcap, layouts
# --------------------------------------------------------------------------
PREFILL_SWEEP = []
for dt, D in (("f32", 32), ("f32", 64), ("bf16", 64), ("bf16", 128), ("f16", 128), ("bf16", 256),
              ("f16", 32)):
    for (Lq, Lk) in ((64, 64), (200, 200), (37, 300), (300, 130), (129, 129)):
        for W in (1, 2, 3, 63, 64, 65, 127, 128, 129, -1, 100000):
            PREFILL_SWEEP.append((dt, D, Lq, Lk, W))


def _prefill_case(dt, D, Lq, Lk, W, seed):
    rng = np.random.default_rng(seed)
    sink_mode = rng.integers(0, 3)
    softcap = float(rng.choice([0.0, 0.0, 5.0]))
    nonpad = None
    if rng.integers(0, 2):
        nonpad = (Lk, int(rng.integers(0, Lk + 1)))
    return Workload("sweep", "prefill", dt, B=2, Hq=4, Hkv=2, D=D, Lq=Lq, Lk=Lk, window=W,
                    softcap=softcap, smooth_softmax=bool(sink_mode == 1),
                    head_sink=bool(sink_mode == 2), nonpad=nonpad, value_scale=0.5 if D > 64 else 1.0,
                    seed=seed)


@pytest.mark.parametrize("dt,D,Lq,Lk,W", PREFILL_SWEEP)
def test_prefill_sweep(gpu, dt, D, Lq, Lk, W):
    seed = zlib.crc32(repr((dt, D, Lq, Lk, W)).encode())
    w = _prefill_case(dt, D, Lq, Lk, W, seed)
    d = generate(w)
    got = gpu_prefill(w, d)
    compare(got, oracle_prefill(w, d), dt, f"prefill {w}")


DECODE_SWEEP = []
for dt, D in (("f32", 64), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("f16", 128)):
    for curr in (1, 2, 3, 4, 16, 40):
        for G in (1, 4, 8):
            for W in (-1, 1, 5, 300):
                DECODE_SWEEP.append((dt, D, curr, G, W))


@pytest.mark.parametrize("dt,D,curr,G,W", DECODE_SWEEP)
def test_decode_sweep(gpu, dt, D, curr, G, W):
    seed = zlib.crc32(repr((dt, D, curr, G, W)).encode())
    rng = np.random.default_rng(seed)
    cap = 700
    seqlens = ("list", rng.integers(curr - 1, cap, size=3).tolist())
    sink_mode = rng.integers(0, 3)
    w = Workload("sweep", "decode", dt, B=3, Hq=2 * G, Hkv=2, D=D, Lq=curr, Lk=cap, window=W,
                 softcap=float(rng.choice([0.0, 30.0])), smooth_softmax=bool(sink_mode == 1),
                 head_sink=bool(sink_mode == 2), seqlens=seqlens, seed=seed)
    d = generate(w)
    out, _, _ = gpu_decode(w, d)
    compare(out, oracle_decode(w, d), dt, f"decode {w}")


def test_prefill_bshd_layout(gpu):
    w = Workload("bshd", "prefill", "bf16", B=2, Hq=8, Hkv=2, D=128, Lq=160, Lk=160, window=50,
                 head_sink=True, seed=11)
    d = generate(w)
    got = gpu_prefill(w, d, layout="bshd")
    compare(got, oracle_prefill(w, d), "bf16", "bshd")
    w32 = w.with_(dtype="f32", D=64)
    d = generate(w32)
    compare(gpu_prefill(w32, d, layout="bshd"), oracle_prefill(w32, d), "f32", "bshd f32")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------
def test_prefill_no_keys_and_empty_batch(gpu):
    w = Workload("nokeys", "prefill", "bf16", B=2, Hq=4, Hkv=2, D=128, Lq=70, Lk=70,
                 head_sink=True, nonpad=(0, 70), seed=12)
    d = generate(w)
    got = gpu_prefill(w, d)
    assert torch.count_nonzero(got[0]).item() == 0
    compare(got, oracle_prefill(w, d), "bf16", "nonpad 0")
    # Lk == 0: every row is empty
    plan = make_plan(w.with_(nonpad=None))
    q = d["q"].cuda()
    out = torch.full_like(q, 7.0)
    empty = torch.empty(2, 2, 0, 128, dtype=q.dtype, device="cuda")
    plan.prefill(q, empty, empty, out, head_sink=d["head_sink"].cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    # B == 0 and Lq == 0 are no-ops
    plan.prefill(q[:0], d["k"].cuda()[:0], d["v"].cuda()[:0], head_sink=d["head_sink"].cuda())


def test_prefill_more_queries_than_keys(gpu):
    for dt, D in (("bf16", 128), ("f32", 32)):
        w = Workload("lq>lk", "prefill", dt, B=1, Hq=2, Hkv=1, D=D, Lq=150, Lk=40, window=-1,
                     smooth_softmax=True, seed=13)
        d = generate(w)
        got = gpu_prefill(w, d)
        assert torch.count_nonzero(got[:, :, :110]).item() == 0
        compare(got, oracle_prefill(w, d), dt, "lq>lk")


def test_decode_out_of_range_lengths_give_zeros(gpu):
    w = Workload("badlen", "decode", "bf16", B=3, Hq=8, Hkv=2, D=128, Lq=2, Lk=64, window=-1,
                 seqlens=("list", [0, 63, 64]), seed=14)
    d = generate(w)
    plan = make_plan(w)
    kc, vc = d["k_cache"].cuda().clone(), d["v_cache"].cuda().clone()
    kc0 = kc.clone()
    seq = d["seqlens_k"].cuda()
    plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq)
    out = plan.decode(d["q"].cuda(), kc, vc, seq)
    torch.cuda.synchronize()
    # batch 0: total 1 < curr 2; batch 2: total 65 > capacity 64 -> skipped, zeros
    assert torch.equal(kc[0], kc0[0]) and torch.equal(kc[2], kc0[2])
    assert torch.count_nonzero(out[0]).item() == 0 and torch.count_nonzero(out[2]).item() == 0
    assert torch.count_nonzero(out[1]).item() > 0


def test_stale_and_padded_slots_are_never_read(gpu):
    # decode: NaN in every slot past seqlens_k
    w = Workload("nan", "decode", "bf16", B=2, Hq=8, Hkv=2, D=128, Lq=3, Lk=600, window=100,
                 head_sink=True, seqlens=("list", [200, 550]), seed=15)
    d = generate(w)
    ref, _, _ = gpu_decode(w, d)
    s = d["seqlens_k"].numpy()
    for b in range(w.B):
        d["k_cache"][b, :, s[b] + 1:] = float("nan")
        d["v_cache"][b, :, s[b] + 1:] = float("nan")
    out, _, _ = gpu_decode(w, d)
    assert torch.equal(out, ref)
    # prefill: NaN in every key slot at or past nonpad
    w = Workload("nanp", "prefill", "bf16", B=2, Hq=4, Hkv=2, D=128, Lq=300, Lk=300, window=70,
                 nonpad=(300, 123), seed=16)
    d = generate(w)
    ref = gpu_prefill(w, d)
    d["k"][1, :, 123:] = float("nan")
    d["v"][1, :, 123:] = float("nan")
    assert torch.equal(gpu_prefill(w, d), ref)


def test_repeat_runs_are_bitwise_identical(gpu):
    w = WORKLOADS[3].with_(Lq=1024, Lk=1024, window=300)
    d = generate(w)
    a = gpu_prefill(w, d)
    b = gpu_prefill(w, d)
    assert torch.equal(a, b)
    w = WORKLOADS[2].with_(Lk=1024, seqlens=("uniform", 100, 1024))
    d = generate(w)
    a, _, _ = gpu_decode(w, d)
    b, _, _ = gpu_decode(w, d)
    assert torch.equal(a, b)


def test_decode_workspace_reuse_across_shapes(gpu):
    """One zero-filled workspace serves many decode calls of different shapes
    and plans: each call must leave its arrival counters at zero."""
    import torch as _t
    cases = [
        Workload("reuse", "decode", "bf16", B=3, Hq=8, Hkv=2, D=128, Lq=1, Lk=900, window=-1,
                 smooth_softmax=True, seqlens=("list", [10, 500, 899]), seed=21),
        Workload("reuse", "decode", "bf16", B=2, Hq=16, Hkv=2, D=128, Lq=4, Lk=900, window=100,
                 head_sink=True, seqlens=("list", [3, 700]), seed=22),
        Workload("reuse", "decode", "bf16", B=4, Hq=8, Hkv=4, D=256, Lq=2, Lk=600, window=-1,
                 softcap=20.0, seqlens=("list", [1, 64, 65, 599]), seed=23),
    ]
    plans = [make_plan(w) for w in cases]
    ws = _t.zeros(max(p.workspace_size() for p in plans), dtype=_t.uint8, device="cuda")
    for rep in range(3):
        for w, plan in zip(cases, plans):
            d = generate(w)
            kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
            seq = d["seqlens_k"].cuda()
            plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq)
            out = plan.decode(d["q"].cuda(), kc, vc, seq, workspace=ws,
                              head_sink=None if d["head_sink"] is None else d["head_sink"].cuda())
            _t.cuda.synchronize()
            compare(out, oracle_decode(w, d), "bf16", f"reuse {rep} {w}")


def test_decode_workspace_reuse_more_tiles_after_fewer(gpu):
    """A call with many (batch, KV head, 16-row) tiles after one with few, on the
    same workspace and without clearing it: the arrival counters sit in a
    fixed region at the front, so the larger call never reads the smaller
    call's partial results as counters."""
    import torch as _t
    small = Workload("reuse_s", "decode", "bf16", B=3, Hq=8, Hkv=2, D=128, Lq=1, Lk=600, window=-1,
                     seqlens=("list", [599, 300, 5]), seed=31)
    big = Workload("reuse_b", "decode", "bf16", B=16, Hq=32, Hkv=8, D=128, Lq=1, Lk=600, window=-1,
                   smooth_softmax=True, seqlens=("uniform", 1, 600), seed=32)
    plans = [make_plan(w) for w in (small, big)]
    ws = _t.zeros(max(p.workspace_size() for p in plans), dtype=_t.uint8, device="cuda")
    for rep in range(2):
        for w, plan in zip((small, big), plans):
            d = generate(w)
            kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
            seq = d["seqlens_k"].cuda()
            plan.append_kv(d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq)
            out = plan.decode(d["q"].cuda(), kc, vc, seq, workspace=ws)
            _t.cuda.synchronize()
            compare(out, oracle_decode(w, d), "bf16", f"reuse {rep} {w}")


@pytest.mark.parametrize("B,lengths", [
    (16, "uniform"), (17, "uniform"),
    (8, [0, 1, 2, 5, 3000, 15, 2999, 1]), (3, [3071, 0, 40]),
])
def test_decode_split_modes(gpu, B, lengths):
    """Both ways the decode kernel cuts its work: with at least two workgroups
    per (batch, KV head, 16-row) tile every tile gets whole workgroups in
    proportion to its keys, otherwise the slices are cuts of the flattened key
    list.  On a 256-workgroup grid, 16 * 8 = 128 tiles take the first and
    17 * 8 = 136 the second; the listed lengths make tiles of very different
    sizes (one key up to 3072 keys) under the first."""
    seed = zlib.crc32(repr(("split", B, lengths)).encode())
    rng = np.random.default_rng(seed)
    cap = 3072
    seq = rng.integers(0, 640, size=B).tolist() if lengths == "uniform" else lengths
    Hkv = 8 if lengths == "uniform" else 2
    w = Workload("split", "decode", "bf16", B=B, Hq=4 * Hkv, Hkv=Hkv, D=128, Lq=1, Lk=cap,
                 window=-1, smooth_softmax=True, seqlens=("list", seq), seed=seed)
    d = generate(w)
    out, _, _ = gpu_decode(w, d)
    compare(out, oracle_decode(w, d), "bf16", f"decode {w}")


@pytest.mark.parametrize("B,Hkv,curr", [(32, 16, 16), (33, 16, 16)])
def test_decode_many_row_tiles(gpu, B, Hkv, curr):
    """Many (batch, KV head, 16-row) tiles in one call: 32*16*4 = 2048 tiles is
    the most the matrix-core decode takes in one launch; 33*16*4 goes through
    the one-wave-per-row kernel.  Both must agree with the oracle."""
    seed = zlib.crc32(repr(("tiles", B, Hkv, curr)).encode())
    rng = np.random.default_rng(seed)
    w = Workload("tiles", "decode", "bf16", B=B, Hq=4 * Hkv, Hkv=Hkv, D=64, Lq=curr, Lk=80,
                 window=24, head_sink=True,
                 seqlens=("list", rng.integers(curr - 1, 80, size=B).tolist()), seed=seed)
    d = generate(w)
    out, _, _ = gpu_decode(w, d)
    compare(out, oracle_decode(w, d), "bf16", f"decode {w}")
