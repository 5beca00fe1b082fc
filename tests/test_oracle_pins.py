"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: a
library routine (scipy softmax/logsumexp, torch autograd of
scaled_dot_product_attention), a closed form, a hand-written fixture from
the pages, finite differences, or the structurally different backward route
printed on the "slime" page. CPU only.
"""
import math
import os

import numpy as np
import pytest
import scipy.special as sp
import torch

import oracle as O
from oracle.sink_attention import _slice_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _dense_slice(rng, Lq, Lk, D):
    return _rand(rng, Lq, D), _rand(rng, Lk, D), _rand(rng, Lk, D)


# --- P1: softmax_n with n = 0 is the vanilla softmax ("Flash-Attention-
# Softmax-N" README formula with n = 0) ----------------------------------
def test_n_zero_is_vanilla_softmax():
    rng = np.random.default_rng(10)
    Q, K, V = _dense_slice(rng, 7, 9, 5)
    keep = O.keep_mask(7, 9, causal=True)
    f = _slice_forward(Q, K, V, O.sink_logit_for_n(0), 0.37, keep)
    S = np.where(keep, 0.37 * Q @ K.T, -np.inf)
    ref = sp.softmax(S, axis=1)
    np.testing.assert_allclose(f["out"], ref @ V, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(f["lse"], sp.logsumexp(S, axis=1), rtol=1e-13)
    np.testing.assert_allclose(f["lse"], f["lse_excl"], rtol=1e-14)


def test_softmax_n_helper_matches_definition():
    rng = np.random.default_rng(11)
    x = _rand(rng, 4, 6) * 3
    for n in (0.0, 0.5, 1.0, 3.0):
        lit = np.exp(x) / (n + np.exp(x).sum(axis=1, keepdims=True))
        np.testing.assert_allclose(O.softmax_n(x, n, axis=1), lit, rtol=1e-13)
    np.testing.assert_allclose(O.softmax_n(x, 0.0, axis=1),
                               sp.softmax(x, axis=1), rtol=1e-13)
    assert O.sink_logit_for_n(0) == -np.inf
    assert O.sink_logit_for_n(0.5) == pytest.approx(math.log(0.5))
    with pytest.raises(ValueError):
        O.sink_logit_for_n(-1)


# --- P2: sigmoid identity ("slime" module docstring) ----------------------
@pytest.mark.parametrize("s", [-2.0, 0.0, 1.3])
def test_sigmoid_identity(s):
    rng = np.random.default_rng(12)
    Q, K, V = _dense_slice(rng, 6, 8, 4)
    keep = O.keep_mask(6, 8, causal=False)
    f = _slice_forward(Q, K, V, s, 0.5, keep)
    S = 0.5 * Q @ K.T
    ident = sp.softmax(S, axis=1) * sp.expit(sp.logsumexp(S, axis=1) - s)[:, None]
    np.testing.assert_allclose(f["P"], ident, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(f["out"], ident @ V, rtol=1e-12, atol=1e-14)


# --- P3: rows sum to less than 1 -----------------------------------------
def test_row_sums_below_one():
    rng = np.random.default_rng(13)
    lens_q, lens_k = [3, 5, 4], [5, 2, 4]
    cu_q = np.r_[0, np.cumsum(lens_q)]
    cu_k = np.r_[0, np.cumsum(lens_k)]
    Hq = 3
    q = _rand(rng, cu_q[-1], Hq, 4)
    k = _rand(rng, cu_k[-1], 1, 4)
    ones = np.ones((cu_k[-1], 1, 4))
    sinks = np.array([0.3, -np.inf, 2.0])
    out, lse, _ = O.sink_attention_forward(q, k, ones, cu_q, cu_k, sinks, 0.4,
                                           causal=True)
    rowsum = out[:, :, 0]
    for b in range(3):
        keep = O.keep_mask(lens_q[b], lens_k[b], True)
        for i in range(lens_q[b]):
            t = cu_q[b] + i
            if not keep[i].any():
                assert np.all(rowsum[t] == 0.0)           # zero output row
                assert lse[0, t] == 0.3 and lse[2, t] == 2.0
                assert lse[1, t] == -np.inf
            else:
                assert rowsum[t, 0] < 1.0 and rowsum[t, 2] < 1.0
                assert rowsum[t, 1] == pytest.approx(1.0, abs=1e-14)


# --- P4: the max-stabilised sink formula of the CANN page, evaluated on its
# own, equals the explicit-column form -----------------------------------
def test_cann_formula():
    rng = np.random.default_rng(14)
    Q, K, V = _dense_slice(rng, 5, 7, 3)
    for sink in (-1.0, 0.0, 25.0):            # 25 > max S: m comes from sink
        S = 0.9 * Q @ K.T
        m = np.maximum(sink, S.max(axis=1))
        num = np.exp(S - m[:, None]) @ V
        den = np.exp(S - m[:, None]).sum(axis=1) + np.exp(sink - m)
        f = _slice_forward(Q, K, V, sink, 0.9, np.ones((5, 7), bool))
        np.testing.assert_allclose(f["out"], num / den[:, None], rtol=1e-12,
                                   atol=1e-300)


# --- P5: masks of issue #108108 (golden fixture) ---------------------------
def _read_masks():
    blocks, cur = [], None
    for line in open(os.path.join(GOLDEN, "masks_issue108108.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.split()[0] in ("mask", "topleft"):
            kind, lq, lk = line.split()
            cur = (kind, int(lq), int(lk), [])
            blocks.append(cur)
        else:
            cur[3].append([int(x) for x in line.split()])
    return blocks


def test_masks_golden():
    blocks = _read_masks()
    assert len(blocks) == 5
    for kind, lq, lk, rows in blocks:
        want = np.array(rows, dtype=bool)
        got = (O.keep_mask(lq, lk, True) if kind == "mask"
               else O.keep_mask_top_left(lq, lk))
        np.testing.assert_array_equal(got, want)


def test_alignments_agree_only_when_square():
    for lq, lk in [(3, 3), (6, 6)]:
        np.testing.assert_array_equal(O.keep_mask(lq, lk, True),
                                      O.keep_mask_top_left(lq, lk))
    for lq, lk in [(2, 5), (5, 2), (1, 7)]:
        assert (O.keep_mask(lq, lk, True) != O.keep_mask_top_left(lq, lk)).any()


def test_fully_masked_rows_zero_output():
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 5, 2, 4), _rand(rng, 2, 1, 4), _rand(rng, 2, 1, 4)
    out, lse, _ = O.sink_attention_forward(q, k, v, [0, 5], [0, 2],
                                           np.array([0.7, -np.inf]), 0.5, True)
    assert np.all(out[:3] == 0.0)               # rows 0..2 keep nothing
    assert np.all(lse[0, :3] == 0.7) and np.all(lse[1, :3] == -np.inf)
    assert np.all(out[3:] != 0.0)


# --- P6: LSE ---------------------------------------------------------------
def test_lse_conventions():
    rng = np.random.default_rng(16)
    Q, K, V = _dense_slice(rng, 6, 6, 4)
    keep = O.keep_mask(6, 6, causal=True, win_left=2)
    f = _slice_forward(Q, K, V, 0.8, 0.6, keep)
    S = np.where(keep, 0.6 * Q @ K.T, -np.inf)
    np.testing.assert_allclose(f["lse_excl"], sp.logsumexp(S, axis=1), rtol=1e-14)
    np.testing.assert_allclose(f["lse"], np.logaddexp(f["lse_excl"], 0.8), rtol=1e-14)
    np.testing.assert_allclose(f["p_sink"], np.exp(0.8 - f["lse"]), rtol=1e-13)


# --- P7: gradients vs central finite differences ---------------------------
def _loss(q, k, v, sinks, dout, cu_q, cu_k, causal, wl, wr, scale):
    out, _, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, scale,
                                         causal, wl, wr)
    return float((out * dout).sum())


@pytest.mark.parametrize("mask", [(True, -1, -1), (True, 1, 0), (False, -1, -1),
                                  (False, 1, 1)])
def test_gradients_finite_differences(mask):
    causal, wl, wr = mask
    rng = np.random.default_rng(17)
    lens = [(5, 2), (2, 5), (3, 3)]
    cu_q = np.r_[0, np.cumsum([a for a, _ in lens])]
    cu_k = np.r_[0, np.cumsum([b for _, b in lens])]
    Hq, Hk, D, scale = 4, 2, 4, 0.45
    q = _rand(rng, cu_q[-1], Hq, D)
    k = _rand(rng, cu_k[-1], Hk, D)
    v = _rand(rng, cu_k[-1], Hk, D)
    dout = _rand(rng, cu_q[-1], Hq, D)
    sinks = np.array([0.2, -0.7, 1.1, -np.inf])
    dq, dk, dv, dsink = O.sink_attention_backward(dout, q, k, v, cu_q, cu_k,
                                                  sinks, scale, causal, wl, wr)
    h = 1e-6
    args = dict(cu_q=cu_q, cu_k=cu_k, causal=causal, wl=wl, wr=wr, scale=scale)

    def fd(arr, setter):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a = arr.copy(); a[idx] += h; lp = setter(a)
            a = arr.copy(); a[idx] -= h; lm = setter(a)
            g[idx] = (lp - lm) / (2 * h)
        return g

    gq = fd(q, lambda a: _loss(a, k, v, sinks, dout, **args))
    gk = fd(k, lambda a: _loss(q, a, v, sinks, dout, **args))
    gv = fd(v, lambda a: _loss(q, k, a, sinks, dout, **args))
    finite = np.isfinite(sinks)
    gs = fd(sinks[finite], lambda a: _loss(q, k, v, np.r_[a, sinks[~finite]],
                                           dout, **args))
    for got, want in ((dq, gq), (dk, gk), (dv, gv), (dsink[finite], gs)):
        err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        assert err <= 1e-6, err
    assert dsink[~finite] == 0.0


# --- P8: the backward route printed on the "slime" page: a vanilla
# attention backward fed dO' = sigma*dO and O' = sigma*O_vanilla, with the
# offset gradient -sum (dO . O_vanilla) sigma (1 - sigma) --------------------
def test_slime_backward_route():
    rng = np.random.default_rng(18)
    Lq, Lk, D, scale, s = 6, 9, 5, 0.4, 0.35
    Q, K, V = _dense_slice(rng, Lq, Lk, D)
    dO = _rand(rng, Lq, D)
    keep = O.keep_mask(Lq, Lk, True)
    # vanilla forward
    S = np.where(keep, scale * Q @ K.T, -np.inf)
    lse_v = sp.logsumexp(S, axis=1)
    Pv = np.exp(S - lse_v[:, None])
    Ov = Pv @ V
    sig = sp.expit(lse_v - s)
    # vanilla FlashAttention-style backward on the modified dO / O
    dOm, Om = sig[:, None] * dO, sig[:, None] * Ov
    Dm = (dOm * Om).sum(axis=1)
    dS = Pv * (dOm @ V.T - Dm[:, None])
    dq_route, dk_route, dv_route = scale * dS @ K, scale * dS.T @ Q, Pv.T @ dOm
    doff_route = -((dO * Ov).sum(axis=1) * sig * (1 - sig)).sum()
    dq, dk, dv, dsink = O.sink_attention_backward(
        dO[:, None], Q[:, None], K[:, None], V[:, None], [0, Lq], [0, Lk],
        np.array([s]), scale, True)
    np.testing.assert_allclose(dq[:, 0], dq_route, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk[:, 0], dk_route, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv[:, 0], dv_route, rtol=1e-12, atol=1e-13)
    assert dsink[0] == pytest.approx(doff_route, rel=1e-12)


# --- P9: integer n == n appended zero keys with zero values ("hf-attention-
# normalizers" Important Limitations: virtual logit-0 / value-0 sink) -------
@pytest.mark.parametrize("n", [1, 2, 3])
def test_integer_n_zero_keys(n):
    rng = np.random.default_rng(19)
    Q, K, V = _dense_slice(rng, 5, 7, 4)
    scale = 0.5
    Kz = np.vstack([K, np.zeros((n, 4))])
    Vz = np.vstack([V, np.zeros((n, 4))])
    ref = sp.softmax(scale * Q @ Kz.T, axis=1) @ Vz
    out, lse, _ = O.sink_attention_forward(
        Q[:, None], K[:, None], V[:, None], [0, 5], [0, 7],
        np.array([O.sink_logit_for_n(n)]), scale, causal=False)
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], sp.logsumexp(scale * Q @ Kz.T, axis=1),
                               rtol=1e-13)


# --- P10: torch SDPA (CPU, fp64) over [K; 0], [V; 0] with an additive bias
# column holding the sink; autograd gives dq, dk, dv and dsink ---------------
@pytest.mark.parametrize("mask", [(True, -1, -1), (True, 3, 0), (False, 2, 1)])
def test_torch_sdpa_with_bias_column(mask):
    causal, wl, wr = mask
    rng = np.random.default_rng(20)
    lens = [(6, 6), (3, 8), (7, 4)]
    Hq, Hk, D, scale = 4, 2, 8, 0.3
    cu_q = np.r_[0, np.cumsum([a for a, _ in lens])]
    cu_k = np.r_[0, np.cumsum([b for _, b in lens])]
    q = _rand(rng, cu_q[-1], Hq, D)
    k = _rand(rng, cu_k[-1], Hk, D)
    v = _rand(rng, cu_k[-1], Hk, D)
    dout = _rand(rng, cu_q[-1], Hq, D)
    sinks = np.array([0.1, -1.0, 0.9, 2.5])
    out, lse, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, scale,
                                           causal, wl, wr)
    dq, dk, dv, dsink = O.sink_attention_backward(dout, q, k, v, cu_q, cu_k,
                                                  sinks, scale, causal, wl, wr)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    ts = torch.tensor(sinks, requires_grad=True)
    outs = []
    G = Hq // Hk
    for b, (lq, lk) in enumerate(lens):
        qs = tq[cu_q[b]:cu_q[b + 1]].transpose(0, 1)           # [H, Lq, D]
        ks = tk[cu_k[b]:cu_k[b + 1]].repeat_interleave(G, 1).transpose(0, 1)
        vs = tv[cu_k[b]:cu_k[b + 1]].repeat_interleave(G, 1).transpose(0, 1)
        zeros = torch.zeros(Hq, 1, D, dtype=torch.float64)
        keep = torch.tensor(O.keep_mask(lq, lk, causal, wl, wr))
        bias = torch.where(keep, 0.0, -math.inf).to(torch.float64)
        bias = torch.cat([bias.expand(Hq, lq, lk),
                          ts[:, None, None].expand(Hq, lq, 1)], dim=2)
        o = torch.nn.functional.scaled_dot_product_attention(
            qs, torch.cat([ks, zeros], 1).contiguous(),
            torch.cat([vs, zeros], 1).contiguous(), attn_mask=bias,
            scale=scale)
        outs.append(o.transpose(0, 1))
    tout = torch.cat(outs, 0)
    (tout * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(out, tout.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dsink, ts.grad.numpy(), rtol=1e-10, atol=1e-11)


# --- P11: GQA == MHA with repeated K/V; dk/dv are group sums ---------------
def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(21)
    cu = [0, 5, 9]
    Hq, Hk, D = 6, 2, 4
    q = _rand(rng, 9, Hq, D); k = _rand(rng, 9, Hk, D); v = _rand(rng, 9, Hk, D)
    dout = _rand(rng, 9, Hq, D)
    sinks = rng.standard_normal(Hq)
    kr, vr = np.repeat(k, Hq // Hk, axis=1), np.repeat(v, Hq // Hk, axis=1)
    a = O.sink_attention_backward(dout, q, k, v, cu, cu, sinks, 0.5, True, 2, 0)
    b = O.sink_attention_backward(dout, q, kr, vr, cu, cu, sinks, 0.5, True, 2, 0)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13)
    np.testing.assert_allclose(a[1], b[1].reshape(9, Hk, Hq // Hk, D).sum(2), rtol=1e-12)
    np.testing.assert_allclose(a[2], b[2].reshape(9, Hk, Hq // Hk, D).sum(2), rtol=1e-12)
    np.testing.assert_allclose(a[3], b[3], rtol=1e-13)


# --- P12: varlen == independent sequences; permutation equivariance --------
def test_varlen_independent_and_permutable():
    rng = np.random.default_rng(22)
    lens_q, lens_k = [4, 1, 6], [4, 5, 3]
    cu_q = np.r_[0, np.cumsum(lens_q)]; cu_k = np.r_[0, np.cumsum(lens_k)]
    q = _rand(rng, cu_q[-1], 2, 4); k = _rand(rng, cu_k[-1], 2, 4)
    v = _rand(rng, cu_k[-1], 2, 4); sinks = np.array([0.5, -0.5])
    out, lse, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, 0.5, True)
    for b in range(3):
        o1, l1, _ = O.sink_attention_forward(
            q[cu_q[b]:cu_q[b + 1]], k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]],
            [0, lens_q[b]], [0, lens_k[b]], sinks, 0.5, True)
        np.testing.assert_array_equal(out[cu_q[b]:cu_q[b + 1]], o1)
        np.testing.assert_array_equal(lse[:, cu_q[b]:cu_q[b + 1]], l1)
    perm = [2, 0, 1]
    qp = np.concatenate([q[cu_q[b]:cu_q[b + 1]] for b in perm])
    kp = np.concatenate([k[cu_k[b]:cu_k[b + 1]] for b in perm])
    vp = np.concatenate([v[cu_k[b]:cu_k[b + 1]] for b in perm])
    cqp = np.r_[0, np.cumsum([lens_q[b] for b in perm])]
    ckp = np.r_[0, np.cumsum([lens_k[b] for b in perm])]
    op, _, _ = O.sink_attention_forward(qp, kp, vp, cqp, ckp, sinks, 0.5, True)
    np.testing.assert_array_equal(
        op, np.concatenate([out[cu_q[b]:cu_q[b + 1]] for b in perm]))


# --- P13: window special cases ---------------------------------------------
def test_window_special_cases():
    for lq, lk in [(5, 5), (3, 7), (7, 3)]:
        np.testing.assert_array_equal(O.keep_mask(lq, lk, True, lk + 3, 0),
                                      O.keep_mask(lq, lk, True))
        np.testing.assert_array_equal(O.keep_mask(lq, lk, False, -1, -1),
                                      np.ones((lq, lk), bool))
    # a (1024, 0) causal window keeps 1025 keys on a full row
    assert O.keep_mask(2048, 2048, True, 1024, 0)[2000].sum() == 1025


# --- P14: tile bookkeeping (hand-derived fixture + element counts) --------
def _read_tiles():
    cases, cur = [], None
    letter = {"D": O.DEAD, "P": O.PARTIAL, "F": O.FULL}
    for line in open(os.path.join(GOLDEN, "tiles_small.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case"):
            cur = (tuple(int(x) for x in line.split()[1:]), [])
            cases.append(cur)
        else:
            cur[1].append([letter[c] for c in line.split()])
    return cases


def test_tile_classes_golden():
    cases = _read_tiles()
    assert len(cases) == 8
    for (lq, lk, tq, tk, causal, wl, wr), rows in cases:
        got = O.classify_tiles(lq, lk, tq, tk, bool(causal), wl, wr)
        np.testing.assert_array_equal(got, np.array(rows), err_msg=str((lq, lk)))


def test_items_cover_every_kept_element():
    rng = np.random.default_rng(23)
    for trial in range(20):
        B = int(rng.integers(1, 5))
        lq = rng.integers(0, 40, B); lk = rng.integers(0, 40, B)
        lq[0] = max(lq[0], 1); lk[0] = max(lk[0], 1)
        cu_q = np.r_[0, np.cumsum(lq)]; cu_k = np.r_[0, np.cumsum(lk)]
        causal = bool(rng.integers(0, 2))
        wl = int(rng.integers(-1, 9)); wr = 0 if causal else int(rng.integers(-1, 9))
        tq, tk = int(rng.choice([2, 4, 8])), int(rng.choice([2, 4, 16]))
        items = O.forward_items(cu_q, cu_k, tq, tk, causal, wl, wr)
        assert len(items) == sum(-(-int(x) // tq) for x in lq)
        covered = 0
        for b, qt, lo, hi, flo, fhi in items:
            keep = O.keep_mask(lq[b], lk[b], causal, wl, wr)
            rows = keep[qt * tq:(qt + 1) * tq]
            covered += rows[:, lo * tk:hi * tk].sum()
            assert rows[:, :lo * tk].sum() == 0 and rows[:, hi * tk:].sum() == 0
            assert lo <= flo <= fhi <= max(hi, lo)
            blk = rows[:, flo * tk:fhi * tk]
            if fhi > flo:
                assert blk.shape == (tq, (fhi - flo) * tk) and blk.all()
        assert covered == O.count_kept_pairs(cu_q, cu_k, causal, wl, wr)
        work = {}
        for it in items:
            work[it[0]] = work.get(it[0], 0) + it[3] - it[2]
        keys = [(-work[it[0]], it[0], -(it[3] - it[2]), it[1]) for it in items]
        assert keys == sorted(keys)
        assert len({(it[0], it[1]) for it in items}) == len(items)
        bitems = O.backward_items(cu_q, cu_k, tq, tk, causal, wl, wr)
        covered = 0
        for b, kt, lo, hi, flo, fhi in bitems:
            keep = O.keep_mask(lq[b], lk[b], causal, wl, wr)
            cols = keep[:, kt * tk:(kt + 1) * tk]
            covered += cols[lo * tq:hi * tq].sum()
            assert cols[:lo * tq].sum() == 0 and cols[hi * tq:].sum() == 0
        assert covered == O.count_kept_pairs(cu_q, cu_k, causal, wl, wr)
        ditems, per_seq = O.decode_items(cu_q, cu_k, tk, 4 * tk, causal, wl, wr)
        for b, (first, n) in enumerate(per_seq):
            mine = ditems[first:first + n]
            assert all(it[0] == b for it in mine)
            if lq[b] and lk[b]:
                colkeep = O.keep_mask(lq[b], lk[b], causal, wl, wr).any(0)
                got = np.zeros(lk[b], bool)
                for _, _, a, c in mine:
                    got[a:c] = True
                assert not (colkeep & ~got).any()
        # cutting the sequences of the last half of the span length into
        # one-tile pieces covers the same keys, contiguously, in the same
        # sequence order; the longest sequence keeps its 4-tile pieces
        titems, tper = O.decode_items(cu_q, cu_k, tk, 4 * tk, causal, wl, wr, tk, 50)
        assert sorted(range(len(tper)), key=lambda b: tper[b][0]) == \
            sorted(range(len(per_seq)), key=lambda b: per_seq[b][0])
        for b, (first, n) in enumerate(tper):
            mine, plain = titems[first:first + n], ditems[per_seq[b][0]:per_seq[b][0] + per_seq[b][1]]
            assert (n == 0) == (len(plain) == 0)
            if n:
                assert (mine[0][2], mine[-1][3]) == (plain[0][2], plain[-1][3])
                assert all(x[3] == y[2] for x, y in zip(mine, mine[1:]))
                assert [it[1] for it in mine] == list(range(n)) and all(it[0] == b for it in mine)
        if titems:
            b0 = titems[0][0]
            assert titems[tper[b0][0]:tper[b0][0] + tper[b0][1]] == \
                ditems[per_seq[b0][0]:per_seq[b0][0] + per_seq[b0][1]]
            spans = {b: (ditems[f][2], ditems[f + n - 1][3]) for b, (f, n) in enumerate(per_seq) if n}
            total, before = sum(hi - lo for lo, hi in spans.values()), 0
            for b in sorted(spans, key=lambda b: tper[b][0]):
                if 2 * before >= total:
                    first, n = tper[b]
                    assert all(it[3] - it[2] <= tk for it in titems[first:first + n])
                before += spans[b][1] - spans[b][0]


def test_dsink_only_matches_full_backward():
    rng = np.random.default_rng(24)
    cu = [0, 7, 19]
    q = _rand(rng, 19, 4, 8); k = _rand(rng, 19, 2, 8); v = _rand(rng, 19, 2, 8)
    dout = _rand(rng, 19, 4, 8); sinks = np.array([0.3, -0.2, -np.inf, 1.0])
    full = O.sink_attention_backward(dout, q, k, v, cu, cu, sinks, 0.4, True, 3, 0)[3]
    only = O.sink_attention_dsink(dout, q, k, v, cu, cu, sinks, 0.4, True, 3, 0, block_rows=4)
    np.testing.assert_allclose(only, full, rtol=1e-12, atol=1e-15)


def test_gather_paged_hand_example():
    """CANN page, PA_BBND layout: row r of sequence b is slot r % bs of page
    block_table[b, r // bs]. Block size 2, four pages whose slot values name
    (page, slot); sequence 0 uses pages 2 then 0 (3 rows), sequence 1 pages 3
    then 1 (2 rows): the gathered rows are read off by hand."""
    cache = np.array([[[0.0], [1.0]], [[10.0], [11.0]], [[20.0], [21.0]], [[30.0], [31.0]]])
    table = np.array([[2, 0], [3, 1]], np.int32)
    rows, cu = O.gather_paged(cache, table, [3, 2], 2)
    assert cu.tolist() == [0, 3, 5]
    assert rows[:, 0].tolist() == [20.0, 21.0, 0.0, 30.0, 31.0]


def test_gather_paged_inverts_a_page_scatter():
    """Rows written into pages one by one (a loop written here, slot by slot)
    come back in order, for a random page permutation, block sizes that do
    and do not divide the lengths, and an empty sequence."""
    rng = np.random.default_rng(11)
    for bs in (1, 3, 16):
        lens = [5, 0, 17, 16]
        need = [(n + bs - 1) // bs for n in lens]
        perm = rng.permutation(sum(need) + 2)
        table = np.zeros((len(lens), max(need)), np.int32)
        cache = np.full((len(perm), bs, 2), -1.0)
        at, want = 0, []
        for b, n in enumerate(lens):
            table[b, :need[b]] = perm[at:at + need[b]]
            at += need[b]
            for r in range(n):
                val = rng.standard_normal(2)
                cache[table[b, r // bs], r % bs] = val
                want.append(val)
        rows, cu = O.gather_paged(cache, table, lens, bs)
        assert cu.tolist() == np.concatenate([[0], np.cumsum(lens)]).tolist()
        assert np.array_equal(rows, np.array(want))


def test_merge_partials_hand_example_and_empty_parts():
    """One part holding e^{lse_p} = 3 of mass with out_p = 2, a sink with
    e^s = 1: the merged mass is 4, so lse = ln 4 and out = 2 * 3/4. Parts
    with no kept key (lse_p = -inf) add nothing; with nothing at all the row
    is the fully masked row of issue #108108 (out 0, lse = s)."""
    out, lse = O.merge_partials(np.array([[[[2.0]]], [[[7.0]]]]),
                                np.array([[[math.log(3.0)]], [[-np.inf]]]), [0.0])
    assert np.isclose(lse[0, 0], math.log(4.0), rtol=0, atol=1e-15)
    assert np.isclose(out[0, 0, 0], 1.5, rtol=0, atol=1e-15)
    out, lse = O.merge_partials(np.zeros((2, 1, 2, 3)), np.full((2, 2, 1), -np.inf),
                                [0.25, -np.inf])
    assert np.all(out == 0) and lse[0, 0] == 0.25 and lse[1, 0] == -np.inf


def test_merge_of_key_split_equals_unsplit_attention():
    """Splitting every sequence's keys into disjoint parts, attending each part
    without the sink and merging gives the unsplit attention with the sink:
    three parts of a non-causal problem, and for a decode-shaped causal
    problem a prefix part (every row keeps all of it: non-causal) plus the
    causal suffix (its bottom-right alignment is the original one)."""
    rng = np.random.default_rng(21)
    hq, hk, d = 4, 2, 16
    sinks = rng.standard_normal(hq)
    lq, lk = [3, 5], [40, 23]
    cu_q = np.r_[0, np.cumsum(lq)].astype(np.int32)
    cu_k = np.r_[0, np.cumsum(lk)].astype(np.int32)
    q = rng.standard_normal((cu_q[-1], hq, d))
    k = rng.standard_normal((cu_k[-1], hk, d))
    v = rng.standard_normal((cu_k[-1], hk, d))
    none = np.full(hq, -np.inf)

    def part(bounds, causal):
        idx = np.concatenate([np.arange(cu_k[b] + a, cu_k[b] + c) for b, (a, c) in enumerate(bounds)])
        ck = np.r_[0, np.cumsum([c - a for a, c in bounds])].astype(np.int32)
        o, l, _ = O.sink_attention_forward(q, k[idx], v[idx], cu_q, ck, none, 0.3, causal, -1, -1)
        return o, l

    ref_o, ref_l, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, 0.3, False, -1, -1)
    parts = [part([(0, 10), (0, 7)], False), part([(10, 31), (7, 8)], False),
             part([(31, 40), (8, 23)], False)]
    mo, ml = O.merge_partials([p[0] for p in parts], [p[1] for p in parts], sinks)
    assert np.allclose(mo, ref_o, rtol=0, atol=1e-12) and np.allclose(ml, ref_l, rtol=0, atol=1e-12)

    ref_o, ref_l, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, 0.3, True, -1, -1)
    # rows sit at key positions >= lk - lq, so keys below that are kept by every row
    pre = [(0, lk[b] - lq[b]) for b in range(2)]
    suf = [(lk[b] - lq[b], lk[b]) for b in range(2)]
    parts = [part(pre, False), part(suf, True)]
    mo, ml = O.merge_partials([p[0] for p in parts], [p[1] for p in parts], sinks)
    assert np.allclose(mo, ref_o, rtol=0, atol=1e-12) and np.allclose(ml, ref_l, rtol=0, atol=1e-12)


def test_keep_row_is_a_row_of_keep_mask():
    """The single-row mask used for sampled rows of long sequences is the
    same rule as the full mask, row for row, over causal / window cases
    with Lq < Lk, Lq = Lk and Lq > Lk."""
    for lq, lk in ((5, 9), (7, 7), (9, 4), (1, 13)):
        for causal, wl, wr in ((True, -1, -1), (False, -1, -1), (True, 2, -1), (False, 3, 1),
                               (False, 0, 0)):
            full = O.keep_mask(lq, lk, causal, wl, wr)
            for i in range(lq):
                assert np.array_equal(O.keep_row(i, lq, lk, causal, wl, wr), full[i])


@pytest.mark.parametrize("mask", [(True, -1, -1), (True, 4, 0), (False, 3, 2), (False, -1, -1)])
def test_sampled_rows_equal_full_problem_rows(mask):
    """sink_attention_rows (the oracle behind the sampled-row checks of the
    full-size workloads) returns, for every (token, q-head), exactly the row
    of the full forward (out, lse) and backward (dq): packed batch with empty
    query and key sequences between non-empty ones (a token right after an
    empty sequence belongs to the next non-empty one), GQA (6 q-heads on 2
    kv-heads), windows, and sequences with Lq > Lk and Lq < Lk."""
    causal, wl, wr = mask
    rng = np.random.default_rng(27)
    lens = [(5, 9), (0, 4), (0, 0), (7, 3), (4, 0), (6, 6), (1, 11)]
    Hq, Hk, D, scale = 6, 2, 8, 0.35
    cu_q = np.r_[0, np.cumsum([a for a, _ in lens])]
    cu_k = np.r_[0, np.cumsum([b for _, b in lens])]
    q = _rand(rng, cu_q[-1], Hq, D)
    k = _rand(rng, cu_k[-1], Hk, D)
    v = _rand(rng, cu_k[-1], Hk, D)
    dout = _rand(rng, cu_q[-1], Hq, D)
    sinks = np.array([0.2, -0.7, 1.3, -np.inf, 0.0, 2.1])
    out, lse, _ = O.sink_attention_forward(q, k, v, cu_q, cu_k, sinks, scale, causal, wl, wr)
    dq = O.sink_attention_backward(dout, q, k, v, cu_q, cu_k, sinks, scale, causal, wl, wr)[0]
    rows = [(t, h) for t in range(cu_q[-1]) for h in range(Hq)]
    got = O.sink_attention_rows(q, k, v, cu_q, cu_k, sinks, scale, causal, wl, wr, rows,
                                dout=dout)
    for (t, h), r in zip(rows, got):
        np.testing.assert_allclose(r["out"], out[t, h], rtol=1e-13, atol=1e-15)
        assert (r["lse"] == lse[h, t]) or abs(r["lse"] - lse[h, t]) <= 1e-13 * abs(lse[h, t])
        np.testing.assert_allclose(r["dq"], dq[t, h], rtol=1e-12, atol=1e-14)
    # the checks above see rows of every kind: kept keys, fully masked rows
    # with a sink (lse = s; the sequence with no keys gives them), and with
    # no sink (lse = -inf)
    t_empty = cu_q[4]                       # first row of the (4, 0) sequence
    assert np.isneginf(lse[3, t_empty]) and lse[0, t_empty] == sinks[0]
    assert np.isfinite(lse[3]).any()


# --- kept-pair count, the FLOP basis of every throughput figure, against
# closed forms of the bottom-right aligned masks ("pytorch/pytorch issue
# #108108": the causal diagonal ends in the bottom-right corner; window
# bounds are read as inclusive on both sides) ------------------------------
def _causal_closed_form(Lq, Lk, wl=-1):
    """Row i keeps keys max(0, i + off - wl) .. min(Lk - 1, i + off),
    off = Lk - Lq, summed with integer arithmetic only."""
    off, total = Lk - Lq, 0
    for i in range(Lq):
        hi = min(Lk - 1, i + off)
        lo = 0 if wl < 0 else max(0, i + off - wl)
        total += max(0, hi - lo + 1)
    return total


def test_count_kept_pairs_closed_forms():
    cu = lambda lens: np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    # square causal: L (L + 1) / 2 per sequence
    lens = [1, 7, 64, 300]
    assert O.count_kept_pairs(cu(lens), cu(lens), True, -1, -1) == sum(L * (L + 1) // 2 for L in lens)
    # no mask: Lq Lk, empty sequences included
    lq, lk = [3, 0, 50, 9], [5, 4, 0, 9]
    assert O.count_kept_pairs(cu(lq), cu(lk), False, -1, -1) == sum(a * b for a, b in zip(lq, lk))
    # causal, Lq < Lk: every row keeps off + i + 1 keys, Lq off + Lq (Lq + 1) / 2
    assert O.count_kept_pairs(cu([4]), cu([10]), True, -1, -1) == 4 * 6 + 4 * 5 // 2
    # causal, Lq > Lk: the first Lq - Lk rows keep nothing, then 1 .. Lk
    assert O.count_kept_pairs(cu([10]), cu([4]), True, -1, -1) == 4 * 5 // 2
    # causal with a left window wl on a square sequence of L > wl rows:
    # wl (wl + 1) / 2 + (L - wl)(wl + 1); the GQA window workload's
    # 8192 rows and wl = 1024 give 7,872,000 per (sequence, head)
    L, wl = 8192, 1024
    want = wl * (wl + 1) // 2 + (L - wl) * (wl + 1)
    assert want == 7_872_000
    assert O.count_kept_pairs(cu([L]), cu([L]), True, wl, 0) == want
    # a small sweep against the row-by-row integer form
    rng = np.random.default_rng(11)
    for _ in range(20):
        a, b = (int(x) for x in rng.integers(0, 90, 2))
        w = int(rng.integers(-1, 40))
        assert O.count_kept_pairs(cu([a]), cu([b]), True, w, 0 if w >= 0 else -1) == \
            _causal_closed_form(a, b, w)
