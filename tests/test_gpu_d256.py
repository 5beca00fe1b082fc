"""head_dim 256 ("CANN ops-transformer: flash_attn", q/k/v validation: D in
{64, 128, 256}) through the C ABI: prefill forward and backward, split-KV
decode, paged decode, a padded layout and the context-parallel merge, against
the oracle with the bf16 tolerances. At this width the tiles live in LDS as
two 128-column slices, and the dK/dV kernel walks 32-row query tiles so that
its five stages fit the LDS. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, TOL, dev_sinks, log, max_abs, oracle_inputs, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _fwd_bwd(p, bwd=True, mode=None):
    log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()} "
        f"H={p.num_heads_q}/{p.num_heads_k} D={p.head_dim} dtype={p.dtype} causal={p.causal} "
        f"win=({p.win_left},{p.win_right})")
    g = HipRun(p)
    if mode is not None:
        assert g.plan.mode == mode
    out, lse = g.fwd()
    args = oracle_inputs(p)
    ro, rl, _ = O.sink_attention_forward(*args)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    log(f"  fwd max|d out|={e_out:.3e} max|d lse|={e_lse:.3e} mode={g.plan.mode}")
    tol = TOL[p.dtype]
    assert e_out <= tol["out"] and e_lse <= tol["lse"]
    if not bwd:
        return g
    dq, dk, dv, ds = g.bwd()
    rq, rk, rv, rs = O.sink_attention_backward(p.as_f32("dout"), *args)
    errs = dict(dq=rel_l2(dq, rq), dk=rel_l2(dk, rk), dv=rel_l2(dv, rv), dsink=rel_l2(ds, rs))
    log("  bwd rel-L2 " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert all(v <= tol["grad"] for v in errs.values()), errs
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    return g


def test_d256_bf16_causal_gqa_ragged():
    p = W.make_problem(201, [1, 63, 200, 517, 130], [1, 63, 200, 517, 300], 8, 2, 256,
                       causal=True, name="d256_causal")
    _fwd_bwd(p, mode=0)


def test_d256_backward_is_deterministic():
    p = W.make_problem(207, [700, 130], [700, 400], 8, 2, 256, causal=True, name="d256_det")
    g = HipRun(p)
    g.fwd()
    first = [t.clone() for t in (lambda r: (g.dq, g.dk, g.dv, g.dsink))(g.bwd())]
    for _ in range(2):
        g.bwd()
        for a, b in zip(first, (g.dq, g.dk, g.dv, g.dsink)):
            assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                               b.view(torch.int16) if b.dtype != torch.float32 else b)
    log("d256 backward: three runs equal bit for bit")


def test_d256_fp16_window_unequal_lengths():
    p = W.make_problem(202, [150, 77, 400], [300, 77, 90], 4, 4, 256, dtype="fp16",
                       causal=False, win_left=37, win_right=20, name="d256_fp16_window")
    _fwd_bwd(p, mode=0)


def test_d256_decode_split_kv():
    p = W.make_problem(203, [1, 5, 16, 3], [700, 2600, 4500, 2049], 16, 4, 256, causal=True,
                       sinks=np.float32(math.log(0.5)), name="d256_decode")
    _fwd_bwd(p, bwd=True, mode=1)


def test_d256_paged_decode_equals_contiguous():
    p = W.make_problem(204, [2, 7, 3], [900, 2100, 64], 16, 4, 256, causal=True,
                       name="d256_paged")
    layout = W.paged_layout(p.cu_k, 32, seed=204, spare=3)
    cache = lambda x: torch.from_numpy(W.scatter_to_pages(x, p.cu_k, layout).view(np.int16)).view(
        torch.bfloat16).cuda()
    plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                       layout.num_blocks, p.num_heads_q, p.num_heads_k, p.head_dim, True)
    out, lse = B.forward_paged(plan, to_dev(p, "q"), cache(p.k), cache(p.v), dev_sinks(p),
                               float(p.scale))
    g = _fwd_bwd(p, bwd=False, mode=1)
    assert torch.equal(out.view(torch.int16), g.out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), g.lse.view(torch.int32))
    log("d256 paged: equal to contiguous")


def test_d256_bnsd_padded():
    from tests.test_gpu_layouts import _run
    _run(205, [96, 0, 41], [130, 7, 64], 96, 130, 8, 4, 256, "BNSD", "BSND")


def test_d256_merge_matches_oracle_merge():
    rng = np.random.default_rng(206)
    P, Tq, Hq, D = 3, 40, 4, 256
    outs = rng.standard_normal((P, Tq, Hq, D)).astype(np.float32)
    lses = (rng.standard_normal((P, Hq, Tq)) * 2).astype(np.float32)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    out, lse = B.merge(torch.from_numpy(outs).cuda(), torch.from_numpy(lses).cuda(),
                       torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    ro, rl = O.merge_partials(outs.astype(np.float64), lses.astype(np.float64),
                              sinks.astype(np.float64))
    e_out, e_lse = max_abs(out.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    log(f"d256 merge: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= TOL["fp32"]["out"] and e_lse <= TOL["fp32"]["lse"]
