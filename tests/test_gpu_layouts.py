"""Batch-padded layouts ("CANN ops-transformer: flash_attn", q/k/v
validation: BSND and BNSD; layout matching table: BNSD q may write BSND out;
SeqLengths group: seqused_q / seqused_kv) through the C ABI: forward and
backward against the oracle on the packed sequences of the used lengths.
Padding rows of the inputs hold NaN (any read of them would show), padding
rows of the outputs must keep their prior contents. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import TOL, dev_sinks, dsink_error, log, max_abs, oracle_inputs, rel_l2

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
SENTINEL = 7.0     # exact in every element type


def _dev(arr, dtype):
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(TORCH[dtype]).cuda()


def _unpad(x, lens, layout):
    """[B, S, N, D] / [B, N, S, D] (numpy) -> packed [sum lens, N, D]."""
    if layout == "BNSD":
        x = x.transpose(0, 2, 1, 3)
    return np.concatenate([x[b, :n] for b, n in enumerate(lens)], axis=0)


def _pad_mask(lens, seq, layout):
    """Boolean [B, S, 1, 1] / [B, 1, S, 1] mask of the padding rows."""
    m = np.arange(seq)[None, :] >= np.asarray(lens)[:, None]
    return m[:, :, None, None] if layout == "BSND" else m[:, None, :, None]


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run(seed, used_q, used_k, seq_q, seq_k, hq, hk, D, layout, layout_out=None,
         dtype="bf16", causal=True, wl=-1, wr=-1, with_used=True, sinks="normal",
         bwd=True, expect_mode=None):
    lout = layout_out or layout
    log(f"case padded {layout}->{lout} used_q={list(used_q)} used_k={list(used_k)} "
        f"S=({seq_q},{seq_k}) H={hq}/{hk} D={D} dtype={dtype} causal={causal} "
        f"win=({wl},{wr}) seqused={with_used}")
    p = W.make_problem(seed, used_q, used_k, hq, hk, D, dtype=dtype, causal=causal,
                       win_left=wl, win_right=wr, sinks=sinks, name="padded")
    nb = len(used_q)
    plan = B.PaddedPlan(nb, seq_q, seq_k, used_q if with_used else None,
                        used_k if with_used else None, hq, hk, D, causal, (wl, wr), dtype,
                        layout, lout)
    if expect_mode is not None:
        assert int(plan.meta[14]) == expect_mode
    nan = W.NAN_BITS[dtype]
    q = _dev(W.pad_rows(p.q, p.cu_q, seq_q, layout, nan), dtype)
    k = _dev(W.pad_rows(p.k, p.cu_k, seq_k, layout, nan), dtype)
    v = _dev(W.pad_rows(p.v, p.cu_k, seq_k, layout, nan), dtype)
    sinks_dev = dev_sinks(p) if sinks is not None else None
    out = torch.full(plan.out_shape(), SENTINEL, dtype=TORCH[dtype], device="cuda")
    lse = torch.full((nb, hq, seq_q), SENTINEL, dtype=torch.float32, device="cuda")
    B.forward_padded(plan, q, k, v, sinks_dev, float(p.scale), out, lse)
    torch.cuda.synchronize()

    args = oracle_inputs(p, sinks is not None)
    ro, rl, _ = O.sink_attention_forward(*args)
    o_np, l_np = _f64(out), lse.cpu().numpy().astype(np.float64)
    e_out = max_abs(_unpad(o_np, used_q, lout), ro)
    e_lse = max(max_abs(l_np[b, :, :n], rl[:, p.cu_q[b]:p.cu_q[b + 1]])
                for b, n in enumerate(used_q))
    log(f"  fwd max|d out|={e_out:.3e} max|d lse|={e_lse:.3e} mode={int(plan.meta[14])}")
    tol = TOL[dtype]
    assert e_out <= tol["out"] and e_lse <= tol["lse"]
    mq_out = np.broadcast_to(_pad_mask(used_q, seq_q, lout), o_np.shape)
    assert (o_np[mq_out] == SENTINEL).all(), "forward wrote a padding row of out"
    mq_lse = np.arange(seq_q)[None, None, :] >= np.asarray(used_q)[:, None, None]
    assert (np.broadcast_to(mq_lse, l_np.shape)[...] <= (l_np == SENTINEL)).all()
    if not bwd:
        return

    # the backward must not read padding rows of out / lse / dO either
    out[torch.from_numpy(np.array(mq_out, copy=True)).cuda()] = float("nan")
    lse[torch.from_numpy(np.array(np.broadcast_to(mq_lse, l_np.shape), copy=True)).cuda()] = \
        float("nan")
    dout = _dev(W.pad_rows(p.dout, p.cu_q, seq_q, lout, nan), dtype)
    dq = torch.full_like(q, SENTINEL)
    dk = torch.full_like(k, SENTINEL)
    dv = torch.full_like(v, SENTINEL)
    dq, dk, dv, ds = B.backward_padded(plan, dout, q, k, v, out, lse, sinks_dev,
                                       float(p.scale), dq, dk, dv)
    torch.cuda.synchronize()
    rq, rk, rv, rs = O.sink_attention_backward(p.as_f32("dout"), *args)
    dq_np, dk_np, dv_np = _f64(dq), _f64(dk), _f64(dv)
    errs = dict(dq=rel_l2(_unpad(dq_np, used_q, layout), rq),
                dk=rel_l2(_unpad(dk_np, used_k, layout), rk),
                dv=rel_l2(_unpad(dv_np, used_k, layout), rv))
    if sinks is not None:
        ds_np = ds.cpu().numpy().astype(np.float64)
        if dtype == "fp32":
            errs["dsink_vs_terms"] = dsink_error(ds_np, rs, ro, rl, p.as_f32("dout"), p.sinks)
        else:
            errs["dsink"] = rel_l2(ds_np, rs)
    log("  bwd rel-L2 " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert all(v <= tol["grad"] for v in errs.values()), errs
    mk = _pad_mask(used_k, seq_k, layout)
    mq = _pad_mask(used_q, seq_q, layout)
    assert (dq_np[np.broadcast_to(mq, dq_np.shape)] == SENTINEL).all()
    assert (dk_np[np.broadcast_to(mk, dk_np.shape)] == SENTINEL).all()
    assert (dv_np[np.broadcast_to(mk, dv_np.shape)] == SENTINEL).all()
    for name, a, m in (("dq", dq_np, mq), ("dk", dk_np, mk), ("dv", dv_np, mk)):
        assert np.isfinite(a[~np.broadcast_to(m, a.shape)]).all(), name


def test_bsnd_self_attention_with_padding():
    _run(301, [70, 0, 33, 130], [70, 0, 33, 130], 130, 130, 8, 2, 128, "BSND")


def test_bnsd_unequal_lengths_d64():
    # bottom-right alignment on the used lengths; an empty query side
    _run(302, [200, 17, 0, 64], [300, 5, 40, 1], 200, 300, 4, 4, 64, "BNSD")


def test_bnsd_q_bsnd_out_fp16_window_full_rows():
    _run(303, [96, 96, 96], [160, 160, 160], 96, 160, 8, 4, 128, "BNSD", "BSND",
         dtype="fp16", causal=False, wl=50, wr=10, with_used=False)


def test_bsnd_decode_split_kv_seqused_kv():
    # one query row per sequence against a partly filled cache: the
    # split-KV path with padded keys
    _run(304, [1, 1, 1, 1], [4096, 1, 2000, 3333], 1, 4096, 32, 4, 128, "BSND",
         sinks=np.float32(math.log(0.5)), bwd=True, expect_mode=1)


def test_bnsd_decode_multi_row_no_sink():
    _run(305, [3, 16, 0], [900, 2600, 50], 16, 2600, 16, 4, 128, "BNSD", sinks=None,
         expect_mode=1)


def test_fp32_padded_layouts():
    _run(306, [37, 5, 0], [50, 9, 3], 40, 64, 4, 2, 64, "BNSD", "BSND", dtype="fp32",
         causal=True, wl=20)
    _run(307, [37, 5, 12], [50, 9, 3], 40, 64, 4, 2, 128, "BSND", dtype="fp32",
         causal=False)


def test_padded_autograd_wrapper_matches_direct_calls():
    """learnable_sink_attn_padded: the same bits as the direct padded calls on
    the used rows, zeros on the padding rows of out and of the gradients."""
    used_q, used_k, S_q, S_k = [50, 0, 33], [70, 5, 64], 64, 80
    p = W.make_problem(310, used_q, used_k, 8, 2, 128, causal=True, name="padded_autograd")
    nb = len(used_q)
    q0 = _dev(W.pad_rows(p.q, p.cu_q, S_q, "BSND", 0), "bf16")
    k0 = _dev(W.pad_rows(p.k, p.cu_k, S_k, "BSND", 0), "bf16")
    v0 = _dev(W.pad_rows(p.v, p.cu_k, S_k, "BSND", 0), "bf16")
    do = _dev(W.pad_rows(p.dout, p.cu_q, S_q, "BSND", 0), "bf16")
    sinks = dev_sinks(p)
    uq = torch.tensor(used_q, dtype=torch.int32, device="cuda")
    uk = torch.tensor(used_k, dtype=torch.int32, device="cuda")
    q, k, v = (t.clone().requires_grad_() for t in (q0, k0, v0))
    s = sinks.clone().requires_grad_()
    out = B.learnable_sink_attn_padded(q, k, v, s, float(p.scale), True, layout="BSND",
                                       seqused_q=uq, seqused_kv=uk)
    out.backward(do)
    torch.cuda.synchronize()
    plan = B.PaddedPlan(nb, S_q, S_k, np.array(used_q, np.int32), np.array(used_k, np.int32), 8, 2,
                        128, True, dtype="bf16", layout="BSND")
    ro, rl = B.forward_padded(plan, q0, k0, v0, sinks, float(p.scale),
                              torch.zeros_like(q0), torch.zeros(nb, 8, S_q, device="cuda"))
    rq, rk, rv, rs = B.backward_padded(plan, do, q0, k0, v0, ro, rl, sinks, float(p.scale),
                                       torch.zeros_like(q0), torch.zeros_like(k0),
                                       torch.zeros_like(v0))
    torch.cuda.synchronize()
    bits = lambda t: t.detach().contiguous().view(torch.int16)
    assert torch.equal(bits(out), bits(ro))
    for got, ref in ((q.grad, rq), (k.grad, rk), (v.grad, rv)):
        assert torch.equal(bits(got), bits(ref))
    assert torch.equal(s.grad, rs)
    mq = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(
        _pad_mask(used_q, S_q, "BSND"), tuple(q0.shape)))).cuda()
    assert (out.detach()[mq] == 0).all() and (q.grad[mq] == 0).all()
    log("padded autograd wrapper: equal to the direct calls, padding rows zero")
