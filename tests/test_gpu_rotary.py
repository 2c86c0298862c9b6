"""Rotary position embedding on the GPU (gqa_apply_rotary, gqa_append_kv_rotary)
against the oracle's rotary (oracle.rotary), on the same seeded inputs.

Element bound: the kernel turns each pair in fp32 and rounds once to the row
type, so |gpu - oracle| <= half an ulp of the result (2^-9 relative for
bf16, 2^-12 for f16; 0 for f32) plus the fp32 arithmetic's own error, a few
2^-24 of |a c| + |b s|.  The check uses one full ulp of the type plus 1e-6 of
the pair's magnitude.  Attention after rotary is compared with the usual
tolerances, the oracle's rotated rows rounded to the row type first, as the
API stores them (the cache and q_rot are tensors of that type).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, make_plan
from windowed_gqa_kv_amd.inputs import TORCH_DTYPES, Workload, generate, rotary_tables, to_f64

pytestmark = pytest.mark.gpu

ULP_REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -23}


def _check_turned(got, x, pos, cos, sin, dtype, what):
    want = oracle.rotary.rotate(to_f64(x), pos, to_f64(cos), to_f64(sin))
    g = to_f64(got)
    D = want.shape[-1]
    a, b = np.abs(to_f64(x)[..., : D // 2]), np.abs(to_f64(x)[..., D // 2:])
    mag = np.concatenate([a + b, a + b], axis=-1)
    bound = ULP_REL[dtype] * np.abs(want) + 1e-6 * mag + 1e-30
    err = np.abs(g - want)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: error {worst:.2f} x bound"


def _round(x64, dtype):
    return torch.from_numpy(x64).to(TORCH_DTYPES[dtype]).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f16", 256), ("f32", 32), ("bf16", 8)])
@pytest.mark.parametrize("pos0", [0, 37])
def test_apply_rotary_matches_oracle(gpu, dtype, D, pos0):
    B, H, L = 2, 3, 53  # ragged: 53 rows, 3 heads
    w = Workload("rot", "prefill", dtype, B=B, Hq=H, Hkv=1, D=D, Lq=L, Lk=L, seed=51 + D + pos0)
    x = generate(w)["q"]
    cos, sin = rotary_tables(pos0 + L + 5, D)
    plan = make_plan(w, max_q_len=L, max_kv_len=L)
    out = plan.apply_rotary(x.cuda(), pos0, cos.cuda(), sin.cuda())
    torch.cuda.synchronize()
    _check_turned(out, x, pos0 + np.arange(L), cos, sin, dtype, f"{dtype} D={D} pos0={pos0}")


def test_apply_rotary_in_place_and_strided(gpu):
    D, L = 128, 40
    w = Workload("rot", "prefill", "bf16", B=2, Hq=4, Hkv=1, D=D, Lq=L, Lk=L, seed=61)
    x = generate(w)["q"]
    cos, sin = rotary_tables(L, D)
    plan = make_plan(w)
    xd = x.cuda()
    same = plan.apply_rotary(xd, 0, cos.cuda(), sin.cuda(), out=xd)
    torch.cuda.synchronize()
    assert same.data_ptr() == xd.data_ptr()
    _check_turned(xd, x, np.arange(L), cos, sin, "bf16", "in place")
    # a view into a longer buffer (row stride of the buffer, not of the view)
    big = torch.zeros(2, 4, L + 24, D, dtype=torch.bfloat16, device="cuda")
    big[:, :, 8:8 + L] = x.cuda()
    view = big[:, :, 8:8 + L]
    out = plan.apply_rotary(view, 0, cos.cuda(), sin.cuda())
    torch.cuda.synchronize()
    _check_turned(out, x, np.arange(L), cos, sin, "bf16", "strided view")
    assert not big[:, :, :8].any() and not big[:, :, 8 + L:].any()


DECODE_CASES = [
    # (dtype, B, Hq, Hkv, D, curr, cap, seqlens)
    ("bf16", 4, 16, 4, 128, 1, 300, [0, 299, 150, 17]),
    ("bf16", 3, 8, 2, 256, 4, 200, [3, 199, 64]),
    ("f16", 2, 8, 8, 64, 3, 128, [2, 100]),
    ("f32", 2, 4, 2, 32, 2, 64, [1, 63]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}_D{c[4]}_curr{c[5]}")
def test_append_kv_rotary_then_decode_matches_oracle(gpu, case):
    dtype, B, Hq, Hkv, D, curr, cap, seq = case
    w = Workload("rotdec", "decode", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, Lq=curr, Lk=cap,
                 window=-1 if D != 256 else 90, smooth_softmax=True, seqlens=("list", seq),
                 seed=71 + D + curr)
    d = generate(w)
    cos, sin = rotary_tables(cap, D)
    plan = make_plan(w)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    seq_d = d["seqlens_k"].cuda()
    q_rot = plan.append_kv_rotary(d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, seq_d,
                                  cos.cuda(), sin.cuda())
    out = plan.decode(q_rot, kc, vc, seq_d)
    torch.cuda.synchronize()

    s = np.asarray(seq, dtype=np.int64)
    pos = oracle.rotary.decode_positions(s, curr)[:, None, :]
    _check_turned(q_rot, d["q"], pos, cos, sin, dtype, "q_rot")
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for b in range(B):
        slots = slice(int(s[b]) + 1 - curr, int(s[b]) + 1)
        _check_turned(kc_h[b, :, slots], d["k_new"][b], pos[b], cos, sin, dtype, f"cached K b={b}")
        assert torch.equal(vc_h[b, :, slots], d["v_new"][b])
        keep = torch.ones(cap, dtype=torch.bool)
        keep[slots] = False
        assert torch.equal(kc_h[b][:, keep], d["k_cache"][b][:, keep]), "other K slots changed"
        assert torch.equal(vc_h[b][:, keep], d["v_cache"][b][:, keep]), "other V slots changed"

    # the oracle's step, with the rotated rows stored in the row type as the API stores them
    q_o, kc_o, vc_o = oracle.rotary.append_kv_rotary(
        to_f64(d["k_cache"]), to_f64(d["v_cache"]), to_f64(d["q"]), to_f64(d["k_new"]),
        to_f64(d["v_new"]), s, to_f64(cos), to_f64(sin))
    q_o = _round(q_o, dtype)
    kc_o = _round(kc_o, dtype)
    want = oracle.decode(q_o, kc_o, vc_o, s, scale=w.sm_scale, window=w.window,
                         smooth_softmax=True)
    compare(out, want, dtype, f"decode after rotary {case}")


def test_append_kv_rotary_in_place_and_skipped_batch(gpu):
    """q_rot may be q itself; a batch whose length is out of range is left alone."""
    D, cap, curr = 128, 64, 2
    w = Workload("rotskip", "decode", "bf16", B=3, Hq=8, Hkv=2, D=D, Lq=curr, Lk=cap,
                 seqlens=("list", [10, 64, 0]), seed=81)  # totals 11 (ok), 65 (> cap), 1 (< curr)
    d = generate(w)
    cos, sin = rotary_tables(cap, D)
    plan = make_plan(w)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    q = d["q"].cuda()
    got = plan.append_kv_rotary(q, d["k_new"].cuda(), d["v_new"].cuda(), kc, vc,
                                d["seqlens_k"].cuda(), cos.cuda(), sin.cuda(), q_rot=q)
    torch.cuda.synchronize()
    assert got.data_ptr() == q.data_ptr()
    _check_turned(q[0], d["q"][0], np.array([9, 10])[None, :], cos, sin, "bf16", "in place q")
    assert torch.equal(q[1:].cpu(), d["q"][1:]), "skipped batches' q rows changed"
    assert torch.equal(kc[1:].cpu(), d["k_cache"][1:]) and torch.equal(vc[1:].cpu(), d["v_cache"][1:])


def test_rotary_prompt_then_prefill_matches_oracle(gpu):
    """Prompt on an empty past: Q at positions Lk - Lq + i, K at j, then prefill."""
    w = Workload("rotpf", "prefill", "bf16", B=1, Hq=8, Hkv=2, D=128, Lq=200, Lk=260, window=64,
                 head_sink=True, value_scale=0.5, seed=91)
    d = generate(w)
    cos, sin = rotary_tables(w.Lk, w.D)
    plan = make_plan(w)
    q_r = plan.apply_rotary(d["q"].cuda(), w.Lk - w.Lq, cos.cuda(), sin.cuda())
    k_r = plan.apply_rotary(d["k"].cuda(), 0, cos.cuda(), sin.cuda())
    out = plan.prefill(q_r, k_r, d["v"].cuda(), head_sink=d["head_sink"].cuda())
    torch.cuda.synchronize()
    qo, ko = oracle.rotary.rotate_prefill(to_f64(d["q"]), to_f64(d["k"]), to_f64(cos), to_f64(sin))
    want = oracle.prefill(_round(qo, "bf16"), _round(ko, "bf16"), to_f64(d["v"]), scale=w.sm_scale,
                          window=w.window, head_sink=to_f64(d["head_sink"]))
    compare(out, want, "bf16", "prefill after rotary")


def test_rotary_full_size_long_prompt_sampled(gpu):
    """The long prompt's Q and K (32 x 8192 and 8 x 8192 rows of 128) as the
    benchmark turns them; sampled rows against the oracle, every row against
    the turn's length invariant."""
    from windowed_gqa_kv_amd.inputs import WORKLOADS
    w = WORKLOADS[3]
    d = generate(w)
    cos, sin = rotary_tables(w.Lk, w.D)
    plan = make_plan(w)
    q_r = plan.apply_rotary(d["q"].cuda(), 0, cos.cuda(), sin.cuda())
    k_r = plan.apply_rotary(d["k"].cuda(), 0, cos.cuda(), sin.cuda())
    torch.cuda.synchronize()
    rows = np.r_[0:5, 4094:4099, 8187:8192, np.random.default_rng(3).integers(0, 8192, 32)]
    for name, src, got in (("q", d["q"], q_r), ("k", d["k"], k_r)):
        g = got[:, :, rows].cpu()
        _check_turned(g, src[:, :, rows], rows, cos, sin, "bf16", f"full-size {name}")
        # pair lengths are kept up to the bf16 rounding of each element
        x = src.cuda().float()
        y = got.float()
        h = w.D // 2
        before = x[..., :h] ** 2 + x[..., h:] ** 2
        after = y[..., :h] ** 2 + y[..., h:] ** 2
        assert float(((after - before).abs() / (before + 1e-6)).max()) < 2 * 2.0 ** -7


@pytest.mark.parametrize("dtype,D,Lq,Lk,W,sink,nonpad", [
    ("bf16", 128, 200, 260, 64, True, None),      # bottom-right: rows at positions 60 .. 259
    ("f16", 64, 300, 300, -1, False, (300, 150)),
    ("bf16", 256, 130, 130, 100, True, None),
    ("bf16", 32, 97, 400, -1, False, None),
])
def test_prefill_rotary_equals_apply_rotary_then_prefill(gpu, dtype, D, Lq, Lk, W, sink, nonpad):
    """gqa_prefill_rotary (Q turned while the prefill loads it) against
    gqa_apply_rotary on Q followed by gqa_prefill: bitwise equal; and against
    the oracle's rotary + attention within the tolerances."""
    B = 1 if nonpad is None else len(nonpad)
    w = Workload("rotfused", "prefill", dtype, B=B, Hq=8, Hkv=2, D=D, Lq=Lq, Lk=Lk, window=W,
                 head_sink=sink, nonpad=nonpad, value_scale=0.5, seed=95 + D + Lq)
    d = generate(w)
    cos, sin = rotary_tables(Lk, D)
    plan = make_plan(w)
    cs, sn = cos.cuda(), sin.cuda()
    np_d = None if d["nonpad"] is None else d["nonpad"].cuda()
    sk = None if d["head_sink"] is None else d["head_sink"].cuda()
    k_r = plan.apply_rotary(d["k"].cuda(), 0, cs, sn)
    q_r = plan.apply_rotary(d["q"].cuda(), Lk - Lq, cs, sn)
    want_gpu = plan.prefill(q_r, k_r, d["v"].cuda(), nonpad_kv_seqlen=np_d, head_sink=sk)
    got = plan.prefill_rotary(d["q"].cuda(), k_r, d["v"].cuda(), cs, sn, nonpad_kv_seqlen=np_d, head_sink=sk)
    torch.cuda.synchronize()
    assert torch.equal(got, want_gpu), "fused rotary differs from apply_rotary + prefill"
    qo, ko = oracle.rotary.rotate_prefill(to_f64(d["q"]), to_f64(d["k"]), to_f64(cos), to_f64(sin))
    want = oracle.prefill(_round(qo, dtype), _round(ko, dtype), to_f64(d["v"]), scale=w.sm_scale, window=W,
                          head_sink=to_f64(d["head_sink"]),
                          nonpad_kv_seqlen=None if d["nonpad"] is None else d["nonpad"].numpy())
    compare(got, want, dtype, f"prefill_rotary {dtype} D={D}")


def test_prefill_rotary_full_size_long_prompt(gpu):
    """The long prompt (32 x 8192 rows, window 4096) with Q turned inside the
    prefill: bitwise equal to the two-pass path."""
    from windowed_gqa_kv_amd.inputs import WORKLOADS
    w = WORKLOADS[3]
    d = generate(w)
    cos, sin = (t.cuda() for t in rotary_tables(w.Lk, w.D))
    plan = make_plan(w)
    k_r = plan.apply_rotary(d["k"].cuda(), 0, cos, sin)
    q = d["q"].cuda()
    a = plan.prefill(plan.apply_rotary(q, 0, cos, sin), k_r, d["v"].cuda())
    b = plan.prefill_rotary(q, k_r, d["v"].cuda(), cos, sin)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_append_kv_rotary_rolling_past_the_tables(gpu):
    """A rolling cache's positions pass the capacity and the host cannot see
    them: rows whose position is at or past the tables are not turned -- their
    K slot and q_rot row are left as they were -- while V is still copied;
    rows inside the tables are turned as usual."""
    W, curr, D = 8, 2, 64
    C = W + curr - 1
    max_pos = 40
    w = Workload("rotpast", "decode", "bf16", B=2, Hq=4, Hkv=2, D=D, Lq=curr, Lk=C, window=W,
                 seqlens=("list", [max_pos, 20]), seed=83)  # batch 0: positions 39, 40; batch 1: 19, 20
    d = generate(w)
    cos, sin = rotary_tables(max_pos, D)
    plan = make_plan(w, rolling_cache=True)
    kc, vc = d["k_cache"].cuda(), d["v_cache"].cuda()
    q = d["q"].cuda()
    q_rot = torch.zeros_like(q)
    plan.append_kv_rotary(q, d["k_new"].cuda(), d["v_new"].cuda(), kc, vc, d["seqlens_k"].cuda(),
                          cos.cuda(), sin.cuda(), q_rot=q_rot)
    torch.cuda.synchronize()
    # batch 0, token 0 at position 39 (inside the tables), token 1 at 40 (past them)
    s39, s40 = 39 % C, 40 % C
    _check_turned(kc[0, :, s39].cpu()[None, :, None], d["k_new"][0, :, 0][None, :, None], np.array([39]), cos, sin,
                  "bf16", "K inside the tables")
    assert torch.equal(kc[0, :, s40].cpu(), d["k_cache"][0, :, s40]), "K past the tables was written"
    assert torch.equal(vc[0, :, s39].cpu(), d["v_new"][0, :, 0]) and torch.equal(vc[0, :, s40].cpu(), d["v_new"][0, :, 1])
    assert not q_rot[0, :, 1].any(), "q_rot past the tables was written"
    _check_turned(q_rot[1].cpu(), d["q"][1], np.array([19, 20])[None, :], cos, sin, "bf16", "batch 1 q")
