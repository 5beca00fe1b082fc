"""Seeded input generators: rounding, reproducibility and the workload
recipes (lengths, ranges, shapes)."""
import math

import numpy as np
import pytest
import torch

from softmax_sink_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  3.0e-39, 65504.0], np.float32)])
    ours = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunked_draws_equal_single_draw(monkeypatch):
    a = W._normal(np.random.default_rng(7), 1000, False)
    monkeypatch.setattr(W, "_CHUNK", 64)
    b = W._normal(np.random.default_rng(7), 1000, False)
    np.testing.assert_array_equal(a, b)


def test_make_problem_is_reproducible():
    p1 = W.make_problem(9, [3, 5], [4, 6], 4, 2, 64)
    p2 = W.make_problem(9, [3, 5], [4, 6], 4, 2, 64)
    for n in ("q", "k", "v", "dout", "sinks"):
        np.testing.assert_array_equal(getattr(p1, n), getattr(p2, n))
    assert p1.q.shape == (8, 4, 64) and p1.k.shape == (10, 2, 64)
    assert p1.scale == np.float32(1 / math.sqrt(64))
    sub = p1.sub_batch([1])
    np.testing.assert_array_equal(sub.q, p1.q[3:])
    np.testing.assert_array_equal(sub.cu_k, [0, 6])


def test_named_configs_small():
    c1 = W.config("softmax1_fp32")
    assert c1.dtype == "fp32" and c1.q.shape == (128, 1, 64)
    assert c1.sinks.tolist() == [0.0] and c1.scale == np.float32(0.125)
    assert not c1.causal


def test_length_recipes():
    # lengths only: reproduce the draws without materialising the tensors
    rng = np.random.default_rng(2)
    lens = rng.integers(64, 2049, 16)
    assert lens.min() >= 64 and lens.max() <= 2048
    rng = np.random.default_rng(3)
    tl = W._train_lengths(rng)
    assert tl.sum() == 32768 and tl.min() >= 1024 and tl.max() <= 8192 and len(tl) == 8
    rng = np.random.default_rng(5)
    lq, lk = rng.integers(1, 17, 64), rng.integers(512, 32769, 64)
    assert lq.min() >= 1 and lq.max() <= 16 and lk.min() >= 512 and lk.max() <= 32768
    assert (lq <= lk).all()


def test_pad_rows_places_every_row():
    """Row i of sequence b (packed index cu[b] + i) lands at [b, i] in BSND
    and [b, :, i] in BNSD (the page's (B, S, N, D) / (B, N, S, D) shapes);
    every other row holds the fill value."""
    cu = np.array([0, 3, 3, 8], np.int32)
    T, N, D, S = 8, 2, 4, 6
    x = (np.arange(T * N * D, dtype=np.float32) + 1).reshape(T, N, D)
    bsnd = W.pad_rows(x, cu, S, "BSND", -1.0)
    bnsd = W.pad_rows(x, cu, S, "BNSD", -1.0)
    assert bsnd.shape == (3, S, N, D) and bnsd.shape == (3, N, S, D)
    seen = 0
    for b in range(3):
        for i in range(S):
            for n in range(N):
                live = i < cu[b + 1] - cu[b]
                want = x[cu[b] + i, n] if live else np.full(D, -1.0, np.float32)
                assert (bsnd[b, i, n] == want).all() and (bnsd[b, n, i] == want).all()
                seen += live
    assert seen == T * N
    with pytest.raises(ValueError):
        W.pad_rows(x, cu, S, "TND", 0.0)


def test_scatter_to_pages_cache_layouts():
    """BNBD holds the same (page, slot, head) elements as BBND with the head
    and slot axes swapped (the page's [num_blocks, KV_N, block_size, D])."""
    cu = np.array([0, 20, 21, 60], np.int32)
    x = (np.arange(60 * 2 * 4, dtype=np.float32) + 1).reshape(60, 2, 4)
    lay = W.paged_layout(cu, 16, seed=3, spare=1)
    a = W.scatter_to_pages(x, cu, lay)
    b = W.scatter_to_pages(x, cu, lay, "BNBD")
    assert b.shape == (lay.num_blocks, 2, 16, 4)
    for pg in range(lay.num_blocks):
        for sl in range(16):
            for h in range(2):
                assert (a[pg, sl, h] == b[pg, h, sl]).all()
    with pytest.raises(ValueError):
        W.scatter_to_pages(x, cu, lay, "NZ")
