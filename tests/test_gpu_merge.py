"""Context-parallel merge through the C ABI: the merge kernel against the
oracle's merge on the same partials, and key-split attention (parts
computed without the sink by the forward, then merged) against the unsplit
oracle. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import TOL, log, max_abs, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("part_dtype,out_dtype,D", [
    (torch.float32, torch.float32, 128), (torch.bfloat16, torch.bfloat16, 128),
    (torch.float32, torch.bfloat16, 64)])
def test_merge_kernel_matches_oracle_merge(part_dtype, out_dtype, D):
    rng = np.random.default_rng(31 + D)
    P, Tq, Hq = 5, 77, 6
    outs = rng.standard_normal((P, Tq, Hq, D)).astype(np.float32)
    lses = (rng.standard_normal((P, Hq, Tq)) * 3 + 2).astype(np.float32)
    lses[1, :, ::4] = -np.inf                         # parts with no kept key
    lses[:, 2, 5] = -np.inf                           # a row no part reaches
    sinks = rng.standard_normal(Hq).astype(np.float32)
    sinks[3] = -np.inf
    po = torch.from_numpy(outs).cuda().to(part_dtype)
    log(f"merge P={P} Tq={Tq} Hq={Hq} D={D} parts {part_dtype} -> {out_dtype}")
    out, lse = B.merge(po, torch.from_numpy(lses).cuda(), torch.from_numpy(sinks).cuda(),
                       out_dtype)
    torch.cuda.synchronize()
    ro, rl = O.merge_partials(po.float().cpu().numpy().astype(np.float64), lses.astype(np.float64),
                              sinks.astype(np.float64))
    got = out.float().cpu().numpy().astype(np.float64)
    e_out = max_abs(got, ro)
    e_lse = max_abs(lse.cpu().numpy(), rl)
    log(f"  max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    # the merge itself is fp32 arithmetic: lse to the fp32 bound, and the
    # output to it as well when stored in fp32; a bf16 output can only be
    # one of the two bf16 neighbours of the exact value (synthetic partials
    # here reach |out| > 4, where half a bf16 step alone exceeds 1e-2)
    assert e_lse <= TOL["fp32"]["lse"]
    if out_dtype == torch.float32:
        assert e_out <= TOL["fp32"]["out"]
    else:
        worst = _bf16_merge_error(got, ro, rl, po.float().cpu().numpy().astype(np.float64),
                                  lses.astype(np.float64))
        log(f"  worst error in bf16 steps of the exact value (+ fp32 sum error): {worst:.3f}")
        assert worst <= 1.0


def _bf16_merge_error(got, ro, rl, outs, lses):
    """Largest |got - exact| in units of (one bf16 step of the exact value +
    the fp32 error of the weighted sum). The merge sums P terms w_p o_p in
    fp32 (w_p = e^(lse_p - lse)), so near-cancelling sums carry an absolute
    error of a few fp32 roundings of sum_p w_p |o_p|, which can exceed one
    bf16 step of their tiny result; 16 roundings cover the accumulation and
    the normalisation."""
    w = np.exp(lses - rl[None])                          # [P, H, T]
    scale = np.einsum("pht,pthd->thd", w, np.abs(outs))  # sum_p w_p |o_p|
    mag = np.maximum(np.abs(ro), np.finfo(np.float32).tiny)
    bound = np.exp2(np.floor(np.log2(mag)) - 7) + 16 * 2.0 ** -24 * scale
    return float(np.max(np.abs(got - ro) / bound))


def _split_forward(p, bounds_per_part, causal_per_part, dtype):
    """Each part: keys [a, c) of every sequence, attended without the sink."""
    outs, lses = [], []
    for bounds, causal in zip(bounds_per_part, causal_per_part):
        idx = np.concatenate([np.arange(p.cu_k[b] + a, p.cu_k[b] + c)
                              for b, (a, c) in enumerate(bounds)])
        cu_k = np.r_[0, np.cumsum([c - a for a, c in bounds])].astype(np.int32)
        plan = B.Plan(p.cu_q, cu_k, p.num_heads_q, p.num_heads_k, p.head_dim, causal,
                      (-1, -1), dtype)
        sub = lambda x: torch.from_numpy(np.ascontiguousarray(x[idx]).view(
            np.int16 if dtype == "bf16" else np.float32)).cuda()
        k, v = sub(p.k), sub(p.v)
        if dtype == "bf16":
            k, v = k.view(torch.bfloat16), v.view(torch.bfloat16)
        o, l = B.forward(plan, to_dev(p, "q"), k, v, None, float(p.scale))
        outs.append(o)
        lses.append(l)
    return torch.stack(outs), torch.stack(lses)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_key_split_then_merge_equals_unsplit(dtype):
    # decode-shaped causal batch: a prefix part every row keeps whole
    # (non-causal) and the causal suffix; plus a 3-way non-causal split
    lq, lk = [3, 1, 8, 5], [700, 130, 2100, 64]
    p = W.make_problem(81, lq, lk, 8, 2, 128, dtype=dtype, causal=True, name=f"cp_{dtype}")
    pre = [(0, lk[b] - lq[b]) for b in range(4)]
    suf = [(lk[b] - lq[b], lk[b]) for b in range(4)]
    po, pl = _split_forward(p, [pre, suf], [False, True], dtype)
    out, lse = B.merge(po, pl, torch.from_numpy(p.sinks).cuda())
    torch.cuda.synchronize()
    ro, rl, _ = O.sink_attention_forward(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.cu_q,
                                         p.cu_k, p.sinks.astype(np.float64), float(p.scale),
                                         True, -1, -1)
    e_out = max_abs(out.float().cpu().numpy(), ro)
    e_lse = max_abs(lse.cpu().numpy(), rl)
    log(f"causal prefix+suffix ({dtype}): max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    tol = TOL[dtype]
    assert e_out <= tol["out"] and e_lse <= tol["lse"]

    thirds = [[(0, c // 3), (c // 3, 2 * c // 3), (2 * c // 3, c)] for c in lk]
    parts = [[t[i] for t in thirds] for i in range(3)]
    po, pl = _split_forward(p, parts, [False] * 3, dtype)
    out, lse = B.merge(po, pl, torch.from_numpy(p.sinks).cuda())
    torch.cuda.synchronize()
    ro, rl, _ = O.sink_attention_forward(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.cu_q,
                                         p.cu_k, p.sinks.astype(np.float64), float(p.scale),
                                         False, -1, -1)
    e_out = max_abs(out.float().cpu().numpy(), ro)
    e_lse = max_abs(lse.cpu().numpy(), rl)
    log(f"non-causal thirds ({dtype}): max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= tol["out"] and e_lse <= tol["lse"]


def test_cp_merge_full_size():
    """The merge bench.py times (4 sink-free bf16 partials of 16640 tokens x
    32 heads x D 128, seed 61), checked on 512 sampled tokens (every head)
    against the oracle's merge of the same partials."""
    from softmax_sink_amd import workloads as W
    P, Hq, D = 4, 32, 128
    Tq = W.config("prefill_varlen").total_q
    outs, lses, sinks = W.merge_inputs(61, P, Tq, Hq, D)
    po = torch.from_numpy(outs.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = B.merge(po, torch.from_numpy(lses).cuda(), torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(7).choice(Tq, 512, replace=False))
    ro, rl = O.merge_partials(W.bf16_bits_to_f32(outs[:, idx]).astype(np.float64),
                              lses[:, :, idx].astype(np.float64), sinks.astype(np.float64))
    got = out[torch.from_numpy(idx).cuda()].float().cpu().numpy().astype(np.float64)
    e_lse = max_abs(lse[:, torch.from_numpy(idx).cuda()].cpu().numpy(), rl)
    worst = _bf16_merge_error(got, ro, rl, W.bf16_bits_to_f32(outs[:, idx]).astype(np.float64),
                              lses[:, :, idx].astype(np.float64))
    log(f"cp_merge full size: max|d lse|={e_lse:.3e}, worst error in bf16 steps "
        f"(+ fp32 sum error) {worst:.3f}")
    assert e_lse <= TOL["fp32"]["lse"] and worst <= 1.0
