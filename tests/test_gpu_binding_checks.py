"""The binding refuses tensors that the kernels would address wrongly -- a
host tensor, a strided view, the wrong dtype or shape for the plan -- with a
ValueError raised before anything is launched. Needs a GPU (the plans keep
device copies of the metadata)."""
import numpy as np
import pytest
import torch

from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import dev_sinks, log, to_dev

pytestmark = pytest.mark.gpu


def _packed():
    p = W.make_problem(5, [40, 17], [40, 17], 4, 2, 64, causal=True, name="checks")
    plan = B.Plan(p.cu_q, p.cu_k, 4, 2, 64, True)
    return p, plan, to_dev(p, "q"), to_dev(p, "k"), to_dev(p, "v"), dev_sinks(p)


def test_forward_and_backward_refuse_misfit_tensors():
    p, plan, q, k, v, s = _packed()
    bad = {
        "host q": (q.cpu(), k, v, s),
        "strided q": (q.transpose(0, 1).contiguous().transpose(0, 1), k, v, s),
        "fp16 q": (q.half(), k, v, s),
        "short k": (q, k[:-1], v, s),
        "wrong heads v": (q, k, v.reshape(p.total_k, 1, 128), s),
        "fp64 sinks": (q, k, v, s.double()),
        "short sinks": (q, k, v, s[:2]),
    }
    for name, (qq, kk, vv, ss) in bad.items():
        with pytest.raises(ValueError):
            B.forward(plan, qq, kk, vv, ss, 0.125)
    out, lse = B.forward(plan, q, k, v, s, 0.125)
    dout = torch.randn_like(out)
    with pytest.raises(ValueError):
        B.backward(plan, dout, q, k, v, out, lse.t().contiguous(), s, 0.125)
    with pytest.raises(ValueError):
        B.backward(plan, dout.float(), q, k, v, out, lse, s, 0.125)
    dq, dk, dv, ds = B.backward(plan, dout, q, k, v, out, lse, s, 0.125)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and ds.shape == s.shape


def test_padded_paged_and_merge_refuse_misfit_tensors():
    p = W.make_problem(6, [30, 30], [50, 50], 4, 2, 64, causal=True, name="checks_pad")
    plan = B.PaddedPlan(2, 30, 50, None, None, 4, 2, 64, True, layout="BSND")
    q = to_dev(p, "q").reshape(2, 30, 4, 64)
    k = to_dev(p, "k").reshape(2, 50, 2, 64)
    v = to_dev(p, "v").reshape(2, 50, 2, 64)
    with pytest.raises(ValueError):            # BNSD shapes for a BSND plan
        B.forward_padded(plan, q.transpose(1, 2).contiguous(), k, v, None, 0.125)
    out, lse = B.forward_padded(plan, q, k, v, None, 0.125)
    with pytest.raises(ValueError):
        B.backward_padded(plan, torch.randn_like(out)[:, :-1], q, k, v, out, lse, None, 0.125)

    layout = W.paged_layout(p.cu_k, 16, seed=6)
    pplan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, 16, layout.num_blocks,
                        4, 2, 64, True)
    kc = torch.zeros(layout.num_blocks, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):            # a BNBD-shaped cache for a BBND plan
        B.forward_paged(pplan, to_dev(p, "q"), kc, kc, None, 0.125)

    parts = torch.randn(2, 10, 4, 64, device="cuda").bfloat16()
    with pytest.raises(ValueError):
        B.merge(parts, torch.zeros(2, 10, 4, device="cuda"), None)
    o, l = B.merge(parts, torch.zeros(2, 4, 10, device="cuda"), None)
    torch.cuda.synchronize()
    assert o.shape == (10, 4, 64) and l.shape == (4, 10)


def test_plan_does_not_wait_for_queued_work():
    """Building a plan (metadata on the host, small copies to the device)
    returns while earlier work is still queued: its copies are staged in
    pinned memory instead of waiting for the stream to drain. ~60 ms of
    matrix products are queued first."""
    import time

    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    p = W.make_problem(5, [40, 17, 300], [40, 17, 300], 4, 2, 64, causal=True, name="async")
    b = a @ a                                   # warm both paths up first
    B.Plan(p.cu_q, p.cu_k, 4, 2, 64, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(60):
        b = a @ a
    queued = time.perf_counter() - t0
    t1 = time.perf_counter()
    plan = B.Plan(p.cu_q, p.cu_k, 4, 2, 64, True)
    built = time.perf_counter() - t1
    t2 = time.perf_counter()
    torch.cuda.synchronize()
    drained = time.perf_counter() - t2
    log(f"queued {queued * 1e3:.1f} ms of products; plan built in {built * 1e3:.2f} ms; "
        f"the queue drained {drained * 1e3:.1f} ms later")
    # the queue was still busy after the plan was built, and building it took
    # a small fraction of that time
    assert drained > 0.01, (queued, built, drained)
    assert built < 0.25 * (built + drained), (queued, built, drained)
    assert np.array_equal(plan.meta_dev.cpu().numpy(), plan.meta)
    assert np.array_equal(plan.cu_q.cpu().numpy(), p.cu_q)
    del b


def test_upload_table_kernel_copies_and_refuses_pageable_memory():
    """sink_attn_upload_table moves an int32 table from pinned host memory to
    the device with a kernel: every word arrives (lengths with a ragged tail
    and a 16-byte-multiple), and a pageable host buffer is refused on the
    host before anything is enqueued."""
    import ctypes
    import numpy as np
    import torch
    from softmax_sink_amd import binding as B
    rng = np.random.default_rng(5)
    for n in (1, 3, 4, 1001, 71344):
        host = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, n, dtype=np.int64).astype(np.int32)).pin_memory()
        dev = torch.full((n + 5,), -7, dtype=torch.int32, device="cuda")
        B.sink_attn_upload_table(host, dev, n)
        torch.cuda.synchronize()
        assert torch.equal(dev[:n].cpu(), host) and (dev[n:] == -7).all()
    pageable = np.zeros(64, np.int32)
    dev = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = B.lib().sink_attn_upload_table(pageable.ctypes.data, dev.data_ptr(), 64,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == B.E_INVALID
    with pytest.raises(ValueError):
        B.sink_attn_upload_table(torch.zeros(8, dtype=torch.int32), dev, 8)


@pytest.mark.parametrize("lens_q", [[1, 7, 16, 3], [130, 7, 300, 64]])
def test_forward_reads_only_the_table_prefix(lens_q):
    """The forward calls read the first meta[META_FWD_WORDS] words of the
    device table: with only that prefix copied (the rest of the device buffer
    zero), the forward gives the same bits as with the whole table, in decode
    mode (split-KV items) and in prefill mode (per-query-tile items)."""
    hq, hk, D = 16, 4, 128
    p = W.make_problem(61, lens_q, [5000, 300, 9000, 700], hq, hk, D, causal=True,
                       name="prefix")
    prob = B.make_problem(p.cu_q, p.cu_k, hq, hk, D, True)
    meta, fws, _ = B.sink_attn_metadata(prob, p.cu_q, p.cu_k)
    pre = B.forward_table_words(meta)
    decode = max(lens_q) * (hq // hk) <= 64
    assert int(meta[14]) == (1 if decode else 0) and 56 < pre < len(meta)
    log(f"case prefix: lens_q={lens_q} mode={int(meta[14])} prefix {pre} of {len(meta)} words")
    full = torch.from_numpy(meta).cuda()
    part = torch.zeros_like(full)
    part[:pre] = full[:pre]
    q, k, v, s = to_dev(p, "q"), to_dev(p, "k"), to_dev(p, "v"), dev_sinks(p)
    cq, ck = torch.from_numpy(p.cu_q).cuda(), torch.from_numpy(p.cu_k).cuda()
    res = []
    for m in (full, part):
        out = torch.empty_like(q)
        lse = torch.empty(hq, p.total_q, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(fws, 1), dtype=torch.uint8, device="cuda")
        B.sink_attn_fwd(prob, meta, m, q, k, v, cq, ck, s, float(p.scale), out, lse, ws, fws)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu(), lse.view(torch.int32).cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
