"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element
by element, on seeded inputs that span several tiles with ragged tails, plus
the edge cases of the method. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, TOL, dsink_error, log, max_abs, oracle_inputs, rel_l2

pytestmark = pytest.mark.gpu


def _check(p, with_sink=True, bwd=True, tol=None):
    log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()[:8]} lens_k={np.diff(p.cu_k).tolist()[:8]} "
        f"H={p.num_heads_q}/{p.num_heads_k} D={p.head_dim} causal={p.causal} "
        f"win=({p.win_left},{p.win_right}) dtype={p.dtype} sink={with_sink}")
    tol = tol or TOL[p.dtype]
    g = HipRun(p, with_sink)
    out, lse = g.fwd()
    args = oracle_inputs(p, with_sink)
    ro, rl, _ = O.sink_attention_forward(*args)
    e_out, e_lse = max_abs(out, ro), max_abs(lse.T, rl.T)
    log(f"  fwd max|d out|={e_out:.3e} max|d lse|={e_lse:.3e} mode={g.plan.mode}")
    assert e_out <= tol["out"] and e_lse <= tol["lse"]
    if not bwd:
        return g
    dq, dk, dv, ds = g.bwd()
    rq, rk, rv, rs = O.sink_attention_backward(p.as_f32("dout"), *args)
    errs = dict(dq=rel_l2(dq, rq), dk=rel_l2(dk, rk), dv=rel_l2(dv, rv))
    if with_sink and p.dtype == "fp32":
        errs["dsink_vs_terms"] = dsink_error(ds, rs, ro, rl, p.as_f32("dout"), p.sinks)
    elif with_sink:
        errs["dsink"] = rel_l2(ds, rs)
    log("  bwd rel-L2 " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert all(v <= tol["grad"] for v in errs.values()), errs
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    return g


def test_softmax1_fp32_config():
    _check(W.config("softmax1_fp32"), bwd=True)


def test_fp32_varlen_gqa_window():
    p = W.make_problem(31, [37, 130, 5], [50, 130, 9], 4, 2, 64, dtype="fp32",
                       causal=True, win_left=20, name="fp32_gqa_window")
    _check(p)


def test_fp32_d128_noncausal():
    p = W.make_problem(32, [70, 3], [40, 90], 2, 1, 128, dtype="fp32", causal=False,
                       win_left=-1, win_right=7, name="fp32_d128")
    _check(p)


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_causal_varlen_ragged(D):
    p = W.make_problem(40 + D, [1, 63, 128, 129, 300, 517], [1, 63, 128, 129, 300, 517],
                       4, 4, D, causal=True, name=f"causal_ragged_d{D}")
    _check(p)


def test_bf16_gqa_sliding_window():
    p = W.make_problem(41, [700, 260, 33], [700, 260, 33], 8, 2, 128, causal=True,
                       win_left=100, win_right=0, name="gqa_window")
    _check(p)


def test_bf16_noncausal_two_sided_window_unequal_lengths():
    p = W.make_problem(42, [150, 77, 400], [300, 77, 90], 4, 2, 128, causal=False,
                       win_left=37, win_right=20, name="two_sided_window")
    _check(p)


def test_bf16_bottom_right_unequal_lengths():
    # Lq > Lk leaves the first Lq - Lk rows with no key (zero output, lse = sink)
    p = W.make_problem(43, [5, 300, 64, 200], [200, 100, 64, 3], 4, 4, 128, causal=True,
                       name="bottom_right")
    g = _check(p)
    out = g.out.float().cpu().numpy()
    assert np.all(out[5:5 + 200] == 0.0)          # rows 0..199 of sequence 1
    lse = g.lse.cpu().numpy()
    np.testing.assert_allclose(lse[:, 5:205], np.repeat(p.sinks[:, None], 200, 1), atol=1e-6)


def test_bf16_no_sink_is_plain_attention():
    p = W.make_problem(44, [200, 129], [200, 129], 4, 2, 128, causal=True, name="no_sink")
    _check(p, with_sink=False)


def test_bf16_minus_inf_sinks_and_fully_masked_rows():
    # sinks = -inf and rows with no kept key: out 0, lse -inf, finite gradients
    p = W.make_problem(45, [100, 10], [30, 4], 2, 2, 64, causal=True, sinks=-np.inf,
                       name="neg_inf_sinks")
    g = _check(p)
    lse = g.lse.cpu().numpy()
    assert np.isneginf(lse[:, :70]).all() and np.isneginf(lse[:, 100:106]).all()


def test_bf16_large_sink_absorbs_mass():
    p = W.make_problem(46, [90], [90], 2, 2, 128, causal=True, sinks=30.0, name="big_sink")
    _check(p)


def test_bf16_softmax_n_half():
    p = W.make_problem(47, [257, 31], [257, 31], 4, 4, 128, causal=False,
                       sinks=np.float32(math.log(0.5)), name="softmax_n_0.5")
    _check(p)


def test_bf16_zero_length_sequences():
    p = W.make_problem(48, [0, 77, 0, 140], [12, 77, 0, 150], 4, 2, 128, causal=True,
                       name="zero_len")
    _check(p)


def test_bf16_multi_query_attention():
    # one kv-head for 16 q-heads (the GQA limit): the dK/dV kernel walks 16
    # q-heads per key tile; head count not a multiple of 8 on the q side too
    p = W.make_problem(49, [200, 37, 129], [260, 37, 300], 16, 1, 64, causal=True,
                       win_left=90, name="mqa_d64")
    _check(p)
    p = W.make_problem(52, [70, 9], [70, 140], 12, 1, 128, causal=False, name="mqa_h12")
    _check(p)


def test_bf16_decode_group_at_split_limit():
    # 4 query rows x 16 q-heads per kv-head = 64 rows: the largest group the
    # split-KV path takes; one more row goes to the tiled path
    p = W.make_problem(53, [4, 1, 4], [900, 3000, 64], 32, 2, 128, causal=True,
                       name="decode_limit")
    assert _check(p, bwd=False).plan.mode == 1
    p = W.make_problem(54, [5, 1, 4], [900, 3000, 64], 32, 2, 128, causal=True,
                       name="decode_limit_plus_one")
    assert _check(p, bwd=False).plan.mode == 0


@pytest.mark.parametrize("D", [128, 64])
def test_bf16_decode_split_kv(D):
    # short query groups: split-KV kernel + combine. A small grid: the
    # chunk shrinks to 512 keys (header word 20) so that the 97 items x 8
    # kv-heads fill the chip; chunk boundaries are crossed, and the items
    # make whole groups of 8 (all kv-heads of a chunk on one XCD) and a
    # remainder of 1 (plain order).
    p = W.make_problem(50 + D, [1, 5, 16, 3, 7, 2, 11, 1, 4, 9],
                       [700, 9000, 4500, 2049, 8193, 300, 12000, 4097, 5000, 600], 32, 8, D,
                       causal=True, sinks=np.float32(math.log(0.5)), name=f"decode_d{D}")
    g = _check(p)
    assert g.plan.mode == 1
    assert (int(g.plan.meta[25]), int(g.plan.meta[20])) == (97, 512)   # items, chunk


def test_bf16_decode_long_grid_tail_chunks():
    # a grid of two rounds and more (115 items x 16 kv-heads): 4096-key
    # chunks, the sequences of the last 10% of the span length in 1024-key
    # chunks (header words 20 and 48), and a remainder of 3 items
    rng = np.random.default_rng(77)
    lq, lk = rng.integers(1, 5, 40), rng.integers(2000, 14001, 40)
    p = W.make_problem(78, lq, lk, 32, 16, 128, causal=True, name="decode_tail")
    g = _check(p, bwd=False)
    assert g.plan.mode == 1
    assert [int(g.plan.meta[w]) for w in (25, 20, 48)] == [115, 4096, 1024]


def test_bf16_decode_window_and_no_sink():
    p = W.make_problem(52, [4, 9], [3000, 5000], 16, 4, 128, causal=True, win_left=1500,
                       name="decode_window")
    g = _check(p, with_sink=False)
    assert g.plan.mode == 1


def test_forward_is_deterministic_and_dkdv_too():
    p = W.make_problem(53, [333, 190], [333, 190], 4, 2, 128, causal=True, name="determinism")
    g = HipRun(p)
    o1, l1 = g.fwd()
    d1 = g.bwd()
    o2, l2 = g.fwd()
    d2 = g.bwd()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for a, b in zip(d1, d2):                    # dq, dk, dv, dsink: no atomics anywhere
        assert np.array_equal(a, b)


def test_guard_bands_untouched():
    p = W.make_problem(54, [129, 64], [129, 64], 4, 2, 128, causal=True, name="guard")
    g = HipRun(p)
    pad = 4096
    Tq, Tk, Hq, Hk, D = p.total_q, p.total_k, 4, 2, 128

    def guarded(n, dtype):
        buf = torch.full((n + 2 * pad,), 7.0, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n]

    ob, out = guarded(Tq * Hq * D, torch.bfloat16)
    lb, lse = guarded(Hq * Tq, torch.float32)
    B.sink_attn_fwd(g.plan.problem, g.plan.meta, g.plan.meta_dev, g.q, g.k, g.v, g.plan.cu_q,
                    g.plan.cu_k, g.sinks, g.scale, out, lse)
    dout = torch.randn(Tq, Hq, D, device="cuda").to(torch.bfloat16)
    bufs = [guarded(Tq * Hq * D, torch.bfloat16), guarded(Tk * Hk * D, torch.bfloat16),
            guarded(Tk * Hk * D, torch.bfloat16), guarded(Hq, torch.float32)]
    ws = torch.empty(g.plan.bwd_ws_bytes, dtype=torch.uint8, device="cuda")
    B.sink_attn_bwd(g.plan.problem, g.plan.meta, g.plan.meta_dev, dout, g.q, g.k, g.v, out,
                    lse, g.plan.cu_q, g.plan.cu_k, g.sinks, g.scale, bufs[0][1], bufs[1][1],
                    bufs[2][1], bufs[3][1], ws, g.plan.bwd_ws_bytes)
    torch.cuda.synchronize()
    for buf, _ in [(ob, out), (lb, lse)] + bufs:
        head, tail = buf[:pad].float(), buf[-pad:].float()
        assert (head == 7.0).all() and (tail == 7.0).all()


def test_autograd_wrapper_matches_direct_calls():
    p = W.make_problem(55, [120, 77], [120, 77], 4, 2, 128, causal=True, win_left=50,
                       name="autograd")
    g = HipRun(p)
    out, lse = g.fwd()
    dq, dk, dv, ds = g.bwd()
    q = g.q.clone().requires_grad_(True)
    k = g.k.clone().requires_grad_(True)
    v = g.v.clone().requires_grad_(True)
    s = g.sinks.clone().requires_grad_(True)
    o = B.learnable_sink_attn_varlen(q, k, v, g.plan.cu_q, g.plan.cu_k, 120, 120, s,
                                     float(p.scale), True, (50, 0))
    o.backward(g.dout)
    assert np.array_equal(o.detach().float().cpu().numpy(), out)
    assert rel_l2(q.grad.float().cpu().numpy(), dq) < 1e-3
    assert np.array_equal(k.grad.float().cpu().numpy(), dk)
    assert np.array_equal(s.grad.cpu().numpy(), ds)


@pytest.mark.parametrize("dtype,lens_q", [("bf16", [150, 77, 400]), ("fp32", [60, 7, 90]),
                                          ("bf16", [3, 1, 5])])
def test_int32_max_windows_equal_unbounded(dtype, lens_q):
    """Windows of 2^31 - 1 (non-causal, both sides; causal, left) give the
    same bits as unbounded windows: the host hands such windows to the
    kernels as unbounded, so their 32-bit mask arithmetic cannot wrap. The
    third case takes the split-KV decode path."""
    big = 2 ** 31 - 1
    lens_k = [300, 77, 90]
    for causal, wl, wr in ((False, big, big), (True, big, 0)):
        res = []
        for w in ((wl, wr), (-1, 0 if causal else -1)):
            p = W.make_problem(43, lens_q, lens_k, 4, 2, 64, dtype=dtype, causal=causal,
                               win_left=w[0], win_right=w[1], name="int32_max_window")
            log(f"case int32 max window: dtype={dtype} causal={causal} win={w}")
            g = HipRun(p)
            g.fwd()
            g.bwd()
            res.append([g.out, g.lse, g.dq, g.dk, g.dv, g.dsink])
        bits = lambda t: t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t
        for a, b in zip(*res):
            assert torch.equal(bits(a), bits(b))
