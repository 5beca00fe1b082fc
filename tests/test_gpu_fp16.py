"""fp16 inputs ("CANN ops-transformer: flash_attn", q/k/v validation: float16
and bfloat16) through the same MFMA kernels as bf16: forward and backward,
split-KV decode, paged decode and the context-parallel merge, against the
oracle with the bf16 tolerances. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, TOL, dev_sinks, log, max_abs, oracle_inputs, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _fwd_bwd(p, bwd=True):
    log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()} "
        f"H={p.num_heads_q}/{p.num_heads_k} D={p.head_dim} dtype={p.dtype}")
    g = HipRun(p)
    out, lse = g.fwd()
    assert g.q.dtype == torch.float16
    args = oracle_inputs(p)
    ro, rl, _ = O.sink_attention_forward(*args)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    log(f"  fwd max|d out|={e_out:.3e} max|d lse|={e_lse:.3e} mode={g.plan.mode}")
    tol = TOL["fp16"]
    assert e_out <= tol["out"] and e_lse <= tol["lse"]
    if not bwd:
        return g
    dq, dk, dv, ds = g.bwd()
    rq, rk, rv, rs = O.sink_attention_backward(p.as_f32("dout"), *args)
    errs = dict(dq=rel_l2(dq, rq), dk=rel_l2(dk, rk), dv=rel_l2(dv, rv), dsink=rel_l2(ds, rs))
    log("  bwd rel-L2 " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert all(v <= tol["grad"] for v in errs.values()), errs
    return g


@pytest.mark.parametrize("D", [128, 64])
def test_fp16_causal_gqa_window(D):
    p = W.make_problem(91 + D, [700, 260, 33, 129], [700, 300, 33, 129], 8, 2, D,
                       dtype="fp16", causal=True, win_left=300, name=f"fp16_d{D}")
    _fwd_bwd(p)


def test_fp16_decode_split_kv():
    p = W.make_problem(93, [1, 5, 16, 3], [700, 2600, 4500, 2049], 32, 8, 128, dtype="fp16",
                       causal=True, sinks=np.float32(math.log(0.5)), name="fp16_decode")
    g = _fwd_bwd(p, bwd=False)
    assert g.plan.mode == 1


def test_fp16_paged_decode_equals_contiguous():
    p = W.make_problem(94, [2, 7, 3], [900, 2100, 64], 16, 4, 128, dtype="fp16", causal=True,
                       name="fp16_paged")
    layout = W.paged_layout(p.cu_k, 32, seed=94, spare=3)
    cache = lambda x: torch.from_numpy(W.scatter_to_pages(x, p.cu_k, layout).view(np.int16)).view(
        torch.float16).cuda()
    plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                       layout.num_blocks, p.num_heads_q, p.num_heads_k, p.head_dim, True,
                       dtype="fp16")
    out, lse = B.forward_paged(plan, to_dev(p, "q"), cache(p.k), cache(p.v), dev_sinks(p),
                               float(p.scale))
    g = HipRun(p)
    g.fwd()
    assert torch.equal(out.view(torch.int16), g.out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), g.lse.view(torch.int32))
    ro, rl, _ = O.sink_attention_forward(*oracle_inputs(p))
    e_out = max_abs(out.float().cpu().numpy(), ro)
    e_lse = max_abs(lse.cpu().numpy(), rl)
    log(f"fp16 paged: equal to contiguous; max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= TOL["fp16"]["out"] and e_lse <= TOL["fp16"]["lse"]


def test_fp16_merge_matches_oracle_merge():
    rng = np.random.default_rng(95)
    P, Tq, Hq, D = 3, 50, 4, 128
    outs = (rng.standard_normal((P, Tq, Hq, D)) * 0.5).astype(np.float16)
    lses = (rng.standard_normal((P, Hq, Tq)) * 2).astype(np.float32)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    out, lse = B.merge(torch.from_numpy(outs).cuda(), torch.from_numpy(lses).cuda(),
                       torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    ro, rl = O.merge_partials(outs.astype(np.float64), lses.astype(np.float64),
                              sinks.astype(np.float64))
    got = out.float().cpu().numpy().astype(np.float64)
    e_lse = max_abs(lse.cpu().numpy(), rl)
    mag = np.maximum(np.abs(ro), 2.0 ** -14)
    worst = float(np.max(np.abs(got - ro) / np.exp2(np.floor(np.log2(mag)) - 10)))
    log(f"fp16 merge: max|d lse|={e_lse:.3e}, worst error in fp16 steps {worst:.3f}")
    assert e_lse <= TOL["fp32"]["lse"] and worst <= 1.0
