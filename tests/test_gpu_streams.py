"""Calls are reentrant: two host threads, each on a stream of its own
(default priority), run the forward and backward of one problem and the
split-KV forward of another at the same time, three times over. Each
result must equal, bit for bit, the result of the same call made alone."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, log

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def test_calls_on_two_streams_at_once_equal_calls_alone():
    pa = W.make_problem(96, [300, 1, 700], [300, 40, 900], 8, 2, 128, causal=True, win_left=200,
                        name="streams_train")
    pb = W.make_problem(97, [1, 3, 16, 2], [500, 4000, 2048, 9000], 32, 8, 128, causal=True,
                        name="streams_decode")
    for p in (pa, pb):
        log(f"case {p.name}: lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()}")
    ga, gb = HipRun(pa), HipRun(pb)
    ga.fwd()
    ga.bwd()
    gb.fwd()
    assert gb.plan.mode == 1 and ga.plan.mode == 0
    ref_a = [ga.out, ga.lse, ga.dq, ga.dk, ga.dv, ga.dsink]
    ref_b = [gb.out, gb.lse]
    torch.cuda.synchronize()

    def run_a():
        with torch.cuda.stream(torch.cuda.Stream()):
            res = []
            for _ in range(3):
                out, lse = B.forward(ga.plan, ga.q, ga.k, ga.v, ga.sinks, ga.scale)
                grads = B.backward(ga.plan, ga.dout, ga.q, ga.k, ga.v, out, lse, ga.sinks, ga.scale)
                res.append([out, lse, *grads])
            torch.cuda.current_stream().synchronize()
            return res

    def run_b():
        with torch.cuda.stream(torch.cuda.Stream()):
            res = [list(B.forward(gb.plan, gb.q, gb.k, gb.v, gb.sinks, gb.scale)) for _ in range(6)]
            torch.cuda.current_stream().synchronize()
            return res

    with cf.ThreadPoolExecutor(2) as ex:
        fa, fb = ex.submit(run_a), ex.submit(run_b)
        got_a, got_b = fa.result(), fb.result()
    torch.cuda.synchronize()
    names_a = ("out", "lse", "dq", "dk", "dv", "dsink")
    for r, res in enumerate(got_a):
        for name, want, got in zip(names_a, ref_a, res):
            assert torch.equal(_bits(want), _bits(got)), f"{pa.name} call {r}: {name}"
    for r, res in enumerate(got_b):
        for name, want, got in zip(("out", "lse"), ref_b, res):
            assert torch.equal(_bits(want), _bits(got)), f"{pb.name} call {r}: {name}"
    log("  every concurrent call equals the call made alone, bit for bit")
