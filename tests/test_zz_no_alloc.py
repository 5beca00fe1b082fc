"""The allocation-free backward (sink_attn_bwd_noalloc, through the C ABI)
against the workspace backward (sink_attn_bwd) on the same inputs: two
calls in a row on one GPU, the second on a smaller problem, so that the
second runs on the scratch array the first left behind. Both run the same
kernels in the same order, so every output must agree bit for bit."""
import numpy as np
import pytest
import torch

from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, log

pytestmark = pytest.mark.gpu


def _both(p):
    g = HipRun(p)
    g.fwd()
    g.bwd()                                   # sink_attn_bwd with a workspace
    ref = [g.dq, g.dk, g.dv, g.dsink]
    dq, dk, dv = torch.empty_like(g.q), torch.empty_like(g.k), torch.empty_like(g.v)
    dsink = torch.empty_like(g.sinks)
    for t in (dq, dk, dv):                    # stale values must be overwritten
        t.fill_(float("nan"))
    dsink.fill_(float("nan"))
    plan = g.plan
    B.sink_attn_bwd_noalloc(plan.problem, plan.meta, plan.meta_dev, g.dout, g.q, g.k, g.v,
                            g.out, g.lse, plan.cu_q, plan.cu_k, g.sinks, g.scale, dq, dk, dv,
                            dsink)
    torch.cuda.synchronize()
    return ref, [dq, dk, dv, dsink]


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def test_noalloc_backward_equals_workspace_backward_twice():
    big = W.make_problem(91, [700, 1, 260, 1500], [900, 40, 260, 1500], 8, 2, 128,
                         causal=True, win_left=300, name="noalloc_big")
    small = W.make_problem(92, [33, 5], [70, 5], 4, 4, 64, causal=False, name="noalloc_small")
    for p in (big, small):
        log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} H={p.num_heads_q}/{p.num_heads_k} "
            f"D={p.head_dim}")
        ref, got = _both(p)
        for name, a, b in zip(("dq", "dk", "dv", "dsink"), ref, got):
            assert torch.equal(_bits(a), _bits(b)), name
        log(f"  {p.name}: noalloc backward equals the workspace backward bit for bit")
