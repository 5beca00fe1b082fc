"""Paged-KV forward (the split-KV decode path, and the tiled path for long
query groups, reading pages through a block table) through the C ABI:
against the oracle, which gathers the pages itself, and bit for bit against
the contiguous forward on the same keys and values. Needs an MI355X."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W
from tests.gpu_util import (HipRun, TOL, dev_sinks, log, max_abs, sampled_rows_error,
                            to_dev)

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_paged(p, layout):
    kc = W.scatter_to_pages(p.k, p.cu_k, layout)
    vc = W.scatter_to_pages(p.v, p.cu_k, layout)
    plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                       layout.num_blocks, p.num_heads_q, p.num_heads_k, p.head_dim, p.causal,
                       (p.win_left, p.win_right))
    out, lse = B.forward_paged(plan, to_dev(p, "q"), _bf16_dev(kc), _bf16_dev(vc),
                               dev_sinks(p), float(p.scale))
    torch.cuda.synchronize()
    return kc, vc, out, lse


def _check_paged(p, layout):
    log(f"case {p.name}: bs={layout.block_size} pages={layout.num_blocks} "
        f"lens_q={np.diff(p.cu_q).tolist()[:8]} lens_k={np.diff(p.cu_k).tolist()[:8]} "
        f"H={p.num_heads_q}/{p.num_heads_k} D={p.head_dim}")
    kc, vc, out, lse = _run_paged(p, layout)
    # the contiguous forward on the same data: identical tiles, identical bits
    g = HipRun(p)
    g.fwd()
    same_out = torch.equal(out.view(torch.int16), g.out.view(torch.int16))
    same_lse = torch.equal(lse.view(torch.int32), g.lse.view(torch.int32))
    log(f"  paged == contiguous: out {same_out} lse {same_lse}")
    assert same_out and same_lse
    return kc, vc, out.float().cpu().numpy().astype(np.float64), \
        lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("bs,D", [(16, 128), (48, 128), (64, 64), (1024, 128)])
def test_paged_decode_matches_oracle_and_contiguous(bs, D):
    p = W.make_problem(60 + bs + D, [1, 5, 16, 3, 7], [700, 2600, 4500, 33, 2049], 32, 8, D,
                       causal=True, sinks=np.float32(math.log(0.5)), name=f"paged_bs{bs}_d{D}")
    layout = W.paged_layout(p.cu_k, bs, seed=bs + D, spare=5)
    kc, vc, out, lse = _check_paged(p, layout)
    # oracle on the keys and values it gathers from the pages
    kg, cu_k = O.gather_paged(W.bf16_bits_to_f32(kc), layout.block_table, layout.seqused, bs)
    vg, _ = O.gather_paged(W.bf16_bits_to_f32(vc), layout.block_table, layout.seqused, bs)
    ro, rl, _ = O.sink_attention_forward(p.as_f32("q"), kg, vg, p.cu_q, cu_k,
                                         p.sinks.astype(np.float64), float(p.scale), True,
                                         -1, -1)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    log(f"  vs oracle: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= TOL["bf16"]["out"] and e_lse <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("bs,D", [(16, 128), (48, 128), (1024, 64), (32, 256)])
def test_paged_prefill_matches_oracle_and_contiguous(bs, D):
    # long query groups take the tiled forward; keys past 2048 make it refill
    # its page list in the middle of a work item
    wl = 1500 if bs == 48 else -1
    p = W.make_problem(80 + bs + D, [300, 1, 129, 700], [300, 900, 2500, 4500], 8, 2, D,
                       causal=True, win_left=wl, name=f"paged_prefill_bs{bs}_d{D}")
    layout = W.paged_layout(p.cu_k, bs, seed=80 + bs, spare=4)
    plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                       layout.num_blocks, p.num_heads_q, p.num_heads_k, D, True, (wl, -1))
    assert int(plan.meta[14]) == 0          # the tiled (prefill) schedule
    kc, vc, out, lse = _check_paged(p, layout)
    kg, cu_k = O.gather_paged(W.bf16_bits_to_f32(kc), layout.block_table, layout.seqused, bs)
    vg, _ = O.gather_paged(W.bf16_bits_to_f32(vc), layout.block_table, layout.seqused, bs)
    ro, rl, _ = O.sink_attention_forward(p.as_f32("q"), kg, vg, p.cu_q, cu_k,
                                         p.sinks.astype(np.float64), float(p.scale), True,
                                         wl, -1)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    log(f"  vs oracle: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= TOL["bf16"]["out"] and e_lse <= TOL["bf16"]["lse"]


def test_paged_shared_prefix_pages_and_window():
    # two sequences share their first two pages (a common prompt prefix);
    # sliding window, no sink on some heads
    bs = 16
    p = W.make_problem(71, [3, 4, 2], [200, 150, 90], 16, 4, 128, causal=True, win_left=100,
                       name="paged_shared_prefix")
    p.k[200:232] = p.k[0:32]
    p.v[200:232] = p.v[0:32]
    p.sinks[::3] = -np.inf
    layout = W.paged_layout(p.cu_k, bs, seed=71, spare=2)
    layout.block_table[1, :2] = layout.block_table[0, :2]
    kc, vc, out, lse = _check_paged(p, layout)
    kg, cu_k = O.gather_paged(W.bf16_bits_to_f32(kc), layout.block_table, layout.seqused, bs)
    vg, _ = O.gather_paged(W.bf16_bits_to_f32(vc), layout.block_table, layout.seqused, bs)
    assert np.array_equal(kg, p.as_f32("k"))
    ro, rl, _ = O.sink_attention_forward(p.as_f32("q"), kg, vg, p.cu_q, cu_k,
                                         p.sinks.astype(np.float64), float(p.scale), True,
                                         100, -1)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    log(f"  vs oracle: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert e_out <= TOL["bf16"]["out"] and e_lse <= TOL["bf16"]["lse"]


def test_decode_paged_full_size():
    p = W.config("decode_paged")
    layout = p.meta["paged"]
    log(f"decode_paged: Tq={p.total_q} Tk={p.total_k} pages={layout.num_blocks} "
        f"bs={layout.block_size}")
    kc, vc, out, lse = _check_paged(p, layout)
    s_out, s_lse = sampled_rows_error(p, out, lse, 256, 5)
    log(f"  sampled rows vs oracle: {s_out:.3e} {s_lse:.3e}")
    assert s_out <= TOL["bf16"]["out"] and s_lse <= TOL["bf16"]["lse"]


def test_prefill_paged_full_size():
    p = W.config("prefill_paged")
    layout = p.meta["paged"]
    log(f"prefill_paged: Tq={p.total_q} Tk={p.total_k} pages={layout.num_blocks} "
        f"bs={layout.block_size}")
    kc, vc, out, lse = _check_paged(p, layout)
    s_out, s_lse = sampled_rows_error(p, out, lse, 256, 6)
    log(f"  sampled rows vs oracle: {s_out:.3e} {s_lse:.3e}")
    assert s_out <= TOL["bf16"]["out"] and s_lse <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("lq", [[1, 5, 16, 3], [300, 1, 129, 700]])
def test_paged_bnbd_cache_equals_bbnd(lq):
    """The PA_BNBD cache ([num_blocks, Hk, block_size, D]) gives the same bits
    as the PA_BBND one, on the split-KV and on the tiled path."""
    p = W.make_problem(90 + len(lq) + lq[0], lq, [700, 900, 2500, 4500], 8, 2, 128, causal=True,
                       name="paged_bnbd")
    layout = W.paged_layout(p.cu_k, 32, seed=91, spare=2)
    res = []
    for cl in ("BBND", "BNBD"):
        plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                           layout.num_blocks, p.num_heads_q, p.num_heads_k, p.head_dim, True,
                           cache_layout=cl)
        kc = _bf16_dev(W.scatter_to_pages(p.k, p.cu_k, layout, cl))
        vc = _bf16_dev(W.scatter_to_pages(p.v, p.cu_k, layout, cl))
        out, lse = B.forward_paged(plan, to_dev(p, "q"), kc, vc, dev_sinks(p), float(p.scale))
        torch.cuda.synchronize()
        res.append((out, lse, int(plan.meta[14])))
    log(f"paged BNBD vs BBND, mode {res[0][2]}")
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1].view(torch.int32), res[1][1].view(torch.int32))


@pytest.mark.parametrize("gib", [3.9, 4.2])
def test_paged_cache_past_2_and_4_gib(gib):
    """The used pages sit at the top of a cache of 3.9 GiB (byte offsets past
    2^31) or 4.2 GiB (past 2^32): the 64-bit row addresses of the paged
    transfer reach them, and both the tiled and the split-KV path give the
    contiguous forward's bits."""
    bs, hk, hq, D = 16, 8, 16, 128
    num_blocks = int(gib * 2 ** 30) // (bs * hk * D * 2)
    rng = np.random.default_rng(int(gib * 10))
    for lens_q in ([300, 2, 700], [3, 1, 8]):
        p = W.make_problem(int(gib * 10) + lens_q[0], lens_q, [900, 2500, 700], hq, hk, D,
                           causal=True, name=f"paged_{gib}gib")
        lens_k = np.diff(p.cu_k)
        need = (lens_k + bs - 1) // bs
        top = np.arange(num_blocks - int(need.sum()), num_blocks, dtype=np.int32)
        rng.shuffle(top)
        table = np.zeros((len(lens_k), int(need.max())), np.int32)
        rows_k = np.zeros((int(need.sum()) * bs, hk, D), np.uint16)
        rows_v = np.zeros_like(rows_k)
        at = 0
        for b, n in enumerate(need):
            table[b, :n] = top[at:at + n]
            seg = slice(int(p.cu_k[b]), int(p.cu_k[b + 1]))
            rows_k[at * bs:at * bs + lens_k[b]] = p.k[seg]
            rows_v[at * bs:at * bs + lens_k[b]] = p.v[seg]
            at += int(n)
        kc = torch.zeros(num_blocks, bs, hk, D, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ids = torch.from_numpy(np.concatenate([table[b, :n] for b, n in enumerate(need)])
                               .astype(np.int64)).cuda()
        kc[ids] = _bf16_dev(rows_k).reshape(-1, bs, hk, D)
        vc[ids] = _bf16_dev(rows_v).reshape(-1, bs, hk, D)
        plan = B.PagedPlan(p.cu_q, lens_k, table, bs, num_blocks, hq, hk, D, True)
        log(f"paged cache {gib} GiB ({num_blocks} pages), mode {int(plan.meta[14])}, "
            f"pages {int(top.min())}..{int(top.max())}")
        out, lse = B.forward_paged(plan, to_dev(p, "q"), kc, vc, dev_sinks(p), float(p.scale))
        g = HipRun(p)
        g.fwd()
        assert torch.equal(out.view(torch.int16), g.out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), g.lse.view(torch.int32))
        del kc, vc
        torch.cuda.empty_cache()
