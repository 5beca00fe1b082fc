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
