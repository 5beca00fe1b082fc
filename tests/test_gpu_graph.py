"""The forward (sink_attn_fwd) and the allocation-free backward
(sink_attn_bwd_noalloc) captured together into one HIP graph
(torch.cuda.CUDAGraph, through the C ABI on the capturing stream) and
replayed. Before each replay every output is overwritten with NaN; between
replays the program runs eager calls of the same entry points on another
problem (the noalloc one rewrites the shared scratch array) and synchronises.
Each replay runs the same kernels on the same inputs as the eager calls, so
its outputs must equal the eager results bit for bit."""
import numpy as np
import pytest
import torch

from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, log

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def _noalloc_bwd(run, out, lse, dq, dk, dv, dsink):
    plan = run.plan
    B.sink_attn_bwd_noalloc(plan.problem, plan.meta, plan.meta_dev, run.dout, run.q, run.k,
                            run.v, out, lse, plan.cu_q, plan.cu_k, run.sinks, run.scale, dq, dk,
                            dv, dsink)


def test_forward_and_noalloc_backward_replay_from_a_graph():
    p = W.make_problem(93, [300, 1, 129, 700], [300, 40, 200, 700], 8, 2, 128, causal=True,
                       win_left=250, name="graph")
    other = W.make_problem(94, [77, 150], [90, 150], 4, 4, 64, causal=False, name="graph_eager")
    log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()} "
        f"H={p.num_heads_q}/{p.num_heads_k} D={p.head_dim}")
    g = HipRun(p)
    g.fwd()
    g.bwd()                                   # eager references (the workspace backward)
    ref = [g.out, g.lse, g.dq, g.dk, g.dv, g.dsink]

    plan = g.plan
    out, lse = torch.empty_like(g.out), torch.empty_like(g.lse)
    ws = torch.empty(max(plan.fwd_ws_bytes, 16), dtype=torch.uint8, device=g.q.device)
    dq, dk, dv = torch.empty_like(g.q), torch.empty_like(g.k), torch.empty_like(g.v)
    dsink = torch.empty_like(g.sinks)
    got = [out, lse, dq, dk, dv, dsink]

    def step():
        B.sink_attn_fwd(plan.problem, plan.meta, plan.meta_dev, g.q, g.k, g.v, plan.cu_q,
                        plan.cu_k, g.sinks, g.scale, out, lse, ws, plan.fwd_ws_bytes)
        _noalloc_bwd(g, out, lse, dq, dk, dv, dsink)

    # one eager call on a side stream first: the noalloc entry point looks up
    # its scratch address on its first call on a device
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    log("  captured forward + noalloc backward")

    e = HipRun(other)
    e.fwd()
    e.bwd()
    eo = [torch.empty_like(e.q), torch.empty_like(e.k), torch.empty_like(e.v),
          torch.empty_like(e.sinks)]
    for rep in range(3):
        for t in got:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv", "dsink"), ref, got):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {name}"
        log(f"  replay {rep}: every output equals the eager result bit for bit")
        # eager work between replays, the noalloc backward among it
        e.fwd()
        _noalloc_bwd(e, e.out, e.lse, *eo)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dsink"), (e.dq, e.dk, e.dv, e.dsink), eo):
            assert torch.equal(_bits(a), _bits(b)), f"eager noalloc after replay {rep}: {name}"


def test_split_kv_forward_replays_from_a_graph():
    # short query groups: split-KV kernel, combine and their workspace
    # partials, all inside the graph
    p = W.make_problem(95, [1, 5, 16, 3], [700, 9000, 4500, 2049], 32, 8, 128, causal=True,
                       name="graph_decode")
    log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()}")
    g = HipRun(p)
    g.fwd()
    assert g.plan.mode == 1
    plan = g.plan
    out, lse = torch.empty_like(g.out), torch.empty_like(g.lse)
    ws = torch.empty(max(plan.fwd_ws_bytes, 16), dtype=torch.uint8, device=g.q.device)

    def step():
        B.sink_attn_fwd(plan.problem, plan.meta, plan.meta_dev, g.q, g.k, g.v, plan.cu_q,
                        plan.cu_k, g.sinks, g.scale, out, lse, ws, plan.fwd_ws_bytes)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)                         # the partials are rewritten by every call
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(g.out), _bits(out)), f"replay {rep}: out"
        assert torch.equal(_bits(g.lse), _bits(lse)), f"replay {rep}: lse"
        log(f"  replay {rep}: out and lse equal the eager result bit for bit")
        g.fwd()                                # eager work on the same inputs between replays
