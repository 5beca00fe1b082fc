"""Seeded random sweep over the configuration space, each case checked
against the fp64 oracle (forward and backward): dtype, head_dim, GQA group,
ragged / empty / unequal sequence lengths, causal and window masks, sink
present / absent / -inf, and decode-shaped batches (short query groups take
the split-KV path). The draws are valid problems by the header's checks, so
every case exercises a supported combination. Needs an MI355X."""
import numpy as np
import pytest

from softmax_sink_amd import workloads as W
from tests.gpu_util import log
from tests.test_gpu_parity import _check

N_CASES = 64


def _draw(idx):
    rng = np.random.default_rng(9000 + idx)
    dtype = str(rng.choice(["bf16", "bf16", "fp16", "fp32"]))
    D = int(rng.choice([64, 128] if dtype == "fp32" else [64, 128, 256]))
    hk = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    hq = hk * group
    batch = int(rng.integers(1, 5))
    decode_like = rng.random() < 0.3
    lens_q, lens_k = [], []
    for _ in range(batch):
        lk = int(rng.choice([0, 1, int(rng.integers(2, 70)), int(rng.integers(70, 420))]))
        if decode_like:
            lq = int(rng.integers(1, 9))
        else:
            kind = int(rng.integers(0, 3))
            lq = lk if kind == 0 else int(rng.integers(0, 320))
        lens_q.append(lq)
        lens_k.append(lk)
    if sum(lens_q) == 0:
        lens_q[0] = 5
    if sum(lens_k) == 0:
        lens_k[-1] = 33
    causal = bool(rng.integers(0, 2))
    win_left = int(rng.choice([-1, -1, int(rng.integers(0, 200))]))
    win_right = (int(rng.choice([-1, 0])) if causal
                 else int(rng.choice([-1, -1, int(rng.integers(0, 100))])))
    sink_kind = str(rng.choice(["normal", "normal", "none", "neg_inf"]))
    sinks = -np.inf if sink_kind == "neg_inf" else "normal"
    p = W.make_problem(9000 + idx, lens_q, lens_k, hq, hk, D, dtype=dtype, causal=causal,
                       win_left=win_left, win_right=win_right, sinks=sinks,
                       name=f"sweep{idx}")
    return p, sink_kind != "none"


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(N_CASES))
def test_random_configuration(idx):
    p, with_sink = _draw(idx)
    log(f"sweep case {idx}")
    _check(p, with_sink=with_sink)


def test_sweep_covers_the_space():
    """The draws reach every dtype, head_dim, both modes, GQA and MHA, with
    and without sink and window (host only)."""
    seen = set()
    for idx in range(N_CASES):
        p, with_sink = _draw(idx)
        lq = np.diff(p.cu_q)
        decode = lq.max() * (p.num_heads_q // p.num_heads_k) <= 64
        seen |= {("dtype", p.dtype), ("D", p.head_dim), ("causal", p.causal),
                 ("decode", bool(decode)), ("sink", with_sink),
                 ("window", p.win_left >= 0 or p.win_right > 0),
                 ("gqa", p.num_heads_q > p.num_heads_k)}
    for key in [("dtype", "bf16"), ("dtype", "fp16"), ("dtype", "fp32"), ("D", 64), ("D", 128),
                ("D", 256), ("causal", True), ("causal", False), ("decode", True),
                ("decode", False), ("sink", True), ("sink", False), ("window", True),
                ("gqa", True), ("gqa", False)]:
        assert key in seen, key


# ---------------------------------------------------------------------------
# Paged K/V and batch-padded layouts: the same idea over their own knobs.
# ---------------------------------------------------------------------------
N_PAGED = 24
N_PADDED = 24


def _draw_paged(idx):
    rng = np.random.default_rng(9500 + idx)
    dtype = str(rng.choice(["bf16", "fp16"]))
    D = int(rng.choice([64, 128, 256]))
    hk = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    batch = int(rng.integers(1, 5))
    decode_like = rng.random() < 0.5
    lens_k = [int(rng.choice([1, int(rng.integers(2, 300)), int(rng.integers(300, 3000))]))
              for _ in range(batch)]
    lens_q = [int(rng.integers(1, 9)) if decode_like else int(rng.integers(0, 400))
              for _ in range(batch)]
    if sum(lens_q) == 0:
        lens_q[0] = 3
    causal = bool(rng.integers(0, 2))
    win_left = int(rng.choice([-1, -1, int(rng.integers(0, 1500))]))
    win_right = -1 if causal else int(rng.choice([-1, -1, int(rng.integers(0, 200))]))
    sink_kind = str(rng.choice(["normal", "normal", "none", "neg_inf"]))
    bs = int(rng.choice([16, 32, 48, 64, 112, 256, 1024]))
    cache_layout = str(rng.choice(["BBND", "BNBD"]))
    p = W.make_problem(9500 + idx, lens_q, lens_k, hk * group, hk, D, dtype=dtype,
                       causal=causal, win_left=win_left, win_right=win_right,
                       sinks=-np.inf if sink_kind == "neg_inf" else "normal",
                       name=f"sweep_paged{idx}")
    layout = W.paged_layout(p.cu_k, bs, seed=9500 + idx, spare=int(rng.integers(0, 4)))
    return p, sink_kind != "none", layout, cache_layout


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(N_PAGED))
def test_random_paged(idx):
    """The paged forward equals the contiguous forward bit for bit and the
    oracle within the bf16 bar."""
    import torch

    from softmax_sink_amd import binding as B
    from tests.gpu_util import HipRun, TOL, dev_sinks, max_abs, oracle_inputs, to_dev
    import oracle as O

    p, with_sink, layout, cache_layout = _draw_paged(idx)
    log(f"sweep paged case {idx}: {p.dtype} D={p.head_dim} H={p.num_heads_q}/{p.num_heads_k} "
        f"lens_q={np.diff(p.cu_q).tolist()} lens_k={np.diff(p.cu_k).tolist()} "
        f"causal={p.causal} win=({p.win_left},{p.win_right}) sink={with_sink} "
        f"bs={layout.block_size} pages={layout.num_blocks} cache={cache_layout}")
    tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float16
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()
    plan = B.PagedPlan(p.cu_q, layout.seqused, layout.block_table, layout.block_size,
                       layout.num_blocks, p.num_heads_q, p.num_heads_k, p.head_dim, p.causal,
                       (p.win_left, p.win_right), dtype=p.dtype, cache_layout=cache_layout)
    kc = dev(W.scatter_to_pages(p.k, p.cu_k, layout, cache_layout))
    vc = dev(W.scatter_to_pages(p.v, p.cu_k, layout, cache_layout))
    sinks = dev_sinks(p) if with_sink else None
    out, lse = B.forward_paged(plan, to_dev(p, "q"), kc, vc, sinks, float(p.scale))
    torch.cuda.synchronize()
    g = HipRun(p, with_sink)
    g.fwd()
    same = (torch.equal(out.view(torch.int16), g.out.view(torch.int16)) and
            torch.equal(lse.view(torch.int32), g.lse.view(torch.int32)))
    ro, rl, _ = O.sink_attention_forward(*oracle_inputs(p, with_sink))
    e_out = max_abs(out.float().cpu().numpy().astype(np.float64), ro)
    e_lse = max_abs(lse.cpu().numpy().astype(np.float64), rl)
    log(f"  mode={int(plan.meta[14])} paged == contiguous: {same}; "
        f"max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    assert same
    assert e_out <= TOL[p.dtype]["out"] and e_lse <= TOL[p.dtype]["lse"]


def _draw_padded(idx):
    rng = np.random.default_rng(9700 + idx)
    dtype = str(rng.choice(["bf16", "bf16", "fp16", "fp32"]))
    D = int(rng.choice([64, 128] if dtype == "fp32" else [64, 128, 256]))
    hk = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 5))
    layout, layout_out = [("BSND", "BSND"), ("BNSD", "BNSD"), ("BNSD", "BSND")][
        int(rng.integers(0, 3))]
    decode_like = rng.random() < 0.3
    seq_q = int(rng.integers(1, 9)) if decode_like else int(rng.integers(1, 300))
    seq_k = int(rng.integers(1, 400))
    with_used = bool(rng.random() < 0.7)
    if with_used:
        used_q = [int(rng.integers(0, seq_q + 1)) for _ in range(batch)]
        used_k = [int(rng.integers(0, seq_k + 1)) for _ in range(batch)]
        used_q[int(rng.integers(0, batch))] = seq_q
        used_k[int(rng.integers(0, batch))] = seq_k
    else:
        used_q, used_k = [seq_q] * batch, [seq_k] * batch
    causal = bool(rng.integers(0, 2))
    wl = int(rng.choice([-1, -1, int(rng.integers(0, 150))]))
    wr = -1 if causal else int(rng.choice([-1, -1, int(rng.integers(0, 80))]))
    sinks = "normal" if rng.random() < 0.75 else None
    return dict(seed=9700 + idx, used_q=used_q, used_k=used_k, seq_q=seq_q, seq_k=seq_k,
                hq=hk * group, hk=hk, D=D, layout=layout, layout_out=layout_out,
                dtype=dtype, causal=causal, wl=wl, wr=wr, with_used=with_used, sinks=sinks)


@pytest.mark.gpu
@pytest.mark.parametrize("idx", range(N_PADDED))
def test_random_padded(idx):
    """Forward and backward in a padded layout against the oracle, with NaN
    in the padding rows of the inputs and sentinels in those of the outputs."""
    from tests.test_gpu_layouts import _run

    kw = _draw_padded(idx)
    log(f"sweep padded case {idx}")
    _run(**kw)


def test_paged_and_padded_sweeps_cover_their_space():
    """Host only: the paged draws reach both cache layouts, both modes, every
    head_dim and page spans past 2048 keys; the padded draws reach all three
    layout pairs, every dtype, and both kinds of seqused."""
    from softmax_sink_amd import binding as B

    seen = set()
    for idx in range(N_PAGED):
        p, with_sink, layout, cl = _draw_paged(idx)
        plan_mode = int(B.sink_attn_metadata_paged(
            B.make_problem_paged(p.cu_q, layout.seqused, p.num_heads_q, p.num_heads_k,
                                 p.head_dim, p.causal, p.win_left, p.win_right,
                                 B.dtype_code(p.dtype)),
            B.PagedKV(layout.block_size, layout.block_table.shape[1], layout.num_blocks,
                      B.CACHE_LAYOUTS[cl]),
            p.cu_q, layout.seqused, layout.block_table)[0][14])
        seen |= {("cache", cl), ("mode", plan_mode), ("D", p.head_dim),
                 ("long", int(layout.seqused.max()) > 2048), ("sink", with_sink)}
    for key in [("cache", "BBND"), ("cache", "BNBD"), ("mode", 0), ("mode", 1), ("D", 64),
                ("D", 128), ("D", 256), ("long", True), ("sink", True), ("sink", False)]:
        assert key in seen, key
    seen = set()
    for idx in range(N_PADDED):
        kw = _draw_padded(idx)
        prob = B.make_problem_padded(len(kw["used_q"]), kw["seq_q"], kw["seq_k"],
                                     np.asarray(kw["used_q"], np.int32) if kw["with_used"] else None,
                                     np.asarray(kw["used_k"], np.int32) if kw["with_used"] else None,
                                     kw["hq"], kw["hk"], kw["D"], kw["causal"], kw["wl"], kw["wr"],
                                     B.dtype_code(kw["dtype"]), kw["layout"], kw["layout_out"])
        B.sink_attn_metadata_padded(prob,
                                    np.asarray(kw["used_q"], np.int32) if kw["with_used"] else None,
                                    np.asarray(kw["used_k"], np.int32) if kw["with_used"] else None)
        seen |= {("layout", kw["layout"], kw["layout_out"]), ("dtype", kw["dtype"]),
                 ("used", kw["with_used"])}
    for key in [("layout", "BSND", "BSND"), ("layout", "BNSD", "BNSD"),
                ("layout", "BNSD", "BSND"), ("dtype", "bf16"), ("dtype", "fp16"),
                ("dtype", "fp32"), ("used", True), ("used", False)]:
        assert key in seen, key
