"""Plain, slow, fp64 CPU oracle for attention with a per-head sink logit.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``softmax_sink_amd``) never imports it, and this
package imports nothing from the product path. Inputs are plain arrays; values
that the GPU sees in bf16 or fp32 are passed in already widened to fp64 by the
caller (the seeded generators in ``softmax_sink_amd.workloads`` produce them).

Sources (pages; each function below cites the passage it follows):

* "slime: learnable_softmax_attention.py" -- module docstring (the sink is one
  extra logit column appended to the scaled scores, dropped after the softmax),
  ``_LearnableSoftmaxFlashAttnVarlen.forward`` (THD layout, lse as
  (nheads, total_q) fp32, outputs in the input dtype) and ``.backward``
  (gradient of the offset: minus the sum over tokens of (dO . O_vanilla) times
  sigmoid' of the post-scale), wrapper docstring (window_size = (left, right),
  -1 = no window; default scale 1/sqrt(headdim)).
* "Flash-Attention-Softmax-N (README)" -- introduction: softmax_n(x)_i =
  exp(x_i) / (n + sum_j exp(x_j)), i.e. a sink logit of ln n.
* "CANN ops-transformer: flash_attn" -- Formula section: with a sink,
  m = max(sink, max S) and Attention = sum e^(S-m) V / (sum e^(S-m) + e^(sink-m));
  the returned softmax_lse formula (sink excluded); Constraints (TND layout,
  Q_N % KV_N == 0, cu_seqlens rules).
* "pytorch/pytorch issue #108108 (causal mask alignment)" -- Proposal: the
  causal mask is aligned to the bottom-right corner when seqlen_q != seqlen_kv,
  and a row whose mask is all zero produces a zero output; Benefits: the
  decode example.
* "hf-attention-normalizers 0.1.0 (project description)" -- Important
  Limitations: the softmax1 kernel treats the extra denominator term as a
  virtual logit-0 / value-0 sink and recomputes probabilities in backward;
  Differentiable Paged Attention: the paged path reads K/V pages through a
  block table (the CANN page gives the page layout and the table).

Readings where the pages are silent:

* LSE convention: ``lse`` returned here is sink-INCLUSIVE,
  ln(e^s + sum_kept e^S). ``lse_excl`` (the CANN page's formula) is also
  returned. With s = -inf the two coincide.
* Windows are inclusive key ranges [i+off-left, i+off+right], aligned to the
  bottom-right corner like the causal mask (off = Lk - Lq); causal means
  right = 0.
* GQA: q-head h reads kv-head h // (Hq // Hk).
* The sink is per q-head and is NOT multiplied by the softmax scale.
* A row with no kept key: out = 0; lse = s (or -inf when s = -inf, in which
  case every gradient of that row is 0).

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Masks -- "pytorch/pytorch issue #108108", Proposal (bottom-right alignment;
# all-zero mask row gives zero output); "slime" wrapper docstring and "CANN
# flash_attn" Mask Parameter Group (win_left / win_right, -1 = unbounded).
# ---------------------------------------------------------------------------
def keep_mask(len_q, len_k, causal, win_left=-1, win_right=-1):
    """Boolean [len_q, len_k]; True where query row i may attend to key j.

    Row i sits at key position i + (len_k - len_q) (bottom-right alignment).
    causal: keep j <= that position. win_right >= 0: keep j <= position +
    win_right. win_left >= 0: keep j >= position - win_left. Bounds are
    inclusive.
    """
    i = np.arange(len_q)[:, None]
    j = np.arange(len_k)[None, :]
    pos = i + (len_k - len_q)
    keep = np.ones((len_q, len_k), dtype=bool)
    if causal:
        keep &= j <= pos
    if win_right >= 0:
        keep &= j <= pos + win_right
    if win_left >= 0:
        keep &= j >= pos - win_left
    return keep


def keep_row(i, len_q, len_k, causal, win_left=-1, win_right=-1):
    """Row i of keep_mask (the same rule, issue #108108 Proposal), without
    building the [len_q, len_k] matrix -- for single rows of long sequences."""
    j = np.arange(len_k)
    pos = i + (len_k - len_q)
    keep = np.ones(len_k, dtype=bool)
    if causal:
        keep &= j <= pos
    if win_right >= 0:
        keep &= j <= pos + win_right
    if win_left >= 0:
        keep &= j >= pos - win_left
    return keep


def keep_mask_top_left(len_q, len_k):
    """The older top-left causal alignment (issue #108108, Current Behavior).
    Only used by tests to show the two alignments differ when len_q != len_k."""
    return np.arange(len_k)[None, :] <= np.arange(len_q)[:, None]


# ---------------------------------------------------------------------------
# One (sequence, q-head) slice, dense, with the sink as an explicit column.
# "slime" module docstring: P = softmax([Q K^T * scale, offset])[..., :-1].
# "CANN flash_attn" Formula: m = max(sink, max S); denominators as written.
# ---------------------------------------------------------------------------
def _slice_forward(Q, K, V, sink, scale, keep):
    """Q [Lq,D], K,V [Lk,D] fp64, keep [Lq,Lk]. Returns a dict with
    out [Lq,D], lse [Lq] (sink-inclusive), lse_excl [Lq], P [Lq,Lk],
    p_sink [Lq]."""
    Lq, Lk = keep.shape
    S = scale * (Q @ K.T)
    S = np.where(keep, S, NEG_INF)
    S_ext = np.concatenate([S, np.full((Lq, 1), sink, dtype=np.float64)], axis=1)
    m = S_ext.max(axis=1)
    live = m > NEG_INF
    out = np.zeros((Lq, Q.shape[1]))
    lse = np.full(Lq, NEG_INF)
    P_ext = np.zeros((Lq, Lk + 1))
    if live.any():
        E = np.exp(S_ext[live] - m[live, None])
        Z = E.sum(axis=1)
        P_ext[live] = E / Z[:, None]
        lse[live] = m[live] + np.log(Z)
    P = P_ext[:, :Lk]
    out = P @ V
    # sink-excluded lse, the formula printed for softmax_lse on the CANN page
    has_key = keep.any(axis=1)
    lse_excl = np.full(Lq, NEG_INF)
    if has_key.any():
        Sk = S[has_key]
        mk = Sk.max(axis=1)
        lse_excl[has_key] = np.log(np.exp(Sk - mk[:, None]).sum(axis=1)) + mk
    return {"out": out, "lse": lse, "lse_excl": lse_excl, "P": P,
            "p_sink": P_ext[:, Lk]}


def _slice_backward(dO, Q, K, V, fwd, scale):
    """Gradient of sum(dO * out) for one slice, by the chain rule through the
    extended softmax (the sink column carries a zero value vector, so its
    dP entry is 0). Returns dQ, dK, dV, dsink (scalar).

    This is the analytic gradient of _slice_forward; it is pinned against
    central finite differences and against the "slime" backward recipe
    (vanilla backward fed sigma*dO and sigma*O_vanilla, offset gradient
    -sum (dO . O_vanilla) sigma (1 - sigma))."""
    P, out, p_sink = fwd["P"], fwd["out"], fwd["p_sink"]
    D = (dO * out).sum(axis=1)              # sum_k P_ik dP_ik over real keys
    dP = dO @ V.T
    dS = P * (dP - D[:, None])              # softmax Jacobian, masked P = 0
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    dV = P.T @ dO
    dsink = float(-(p_sink * D).sum())      # sink column: P_sink * (0 - D)
    return dQ, dK, dV, dsink


# ---------------------------------------------------------------------------
# Packed varlen (THD) drivers -- "slime" wrapper docstring: q (total_q,
# nheads, headdim), k/v (total_k, nheads_k, headdim), cu_seqlens (B+1,);
# "CANN flash_attn" Constraints: TND layout, Q_N % KV_N == 0.
# ---------------------------------------------------------------------------
def _check_problem(q, k, v, cu_q, cu_k, sinks):
    Tq, Hq, D = q.shape
    Tk, Hk, Dk = k.shape
    assert v.shape == k.shape and Dk == D
    assert Hq % Hk == 0
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    assert cu_q.shape == cu_k.shape and cu_q[0] == 0 and cu_k[0] == 0
    assert cu_q[-1] == Tq and cu_k[-1] == Tk
    assert np.all(np.diff(cu_q) >= 0) and np.all(np.diff(cu_k) >= 0)
    assert np.asarray(sinks).shape == (Hq,)
    return cu_q, cu_k, Hq // Hk


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _row_blocks(keep, block_rows):
    """Split the rows of a slice into blocks; for each block return the
    contiguous key span that holds every kept key of those rows. Keys
    outside the span are asserted to be masked for those rows."""
    Lq, Lk = keep.shape
    for r0 in range(0, Lq, block_rows):
        r1 = min(Lq, r0 + block_rows)
        cols = np.nonzero(keep[r0:r1].any(axis=0))[0]
        if cols.size == 0:
            j0, j1 = 0, 0
        else:
            j0, j1 = int(cols[0]), int(cols[-1]) + 1
        assert not keep[r0:r1, :j0].any() and not keep[r0:r1, j1:].any()
        yield r0, r1, j0, j1


def sink_attention_forward(q, k, v, cu_q, cu_k, sinks, scale, causal,
                           win_left=-1, win_right=-1, block_rows=512,
                           heads=None):
    """Forward over a packed batch. Returns (out [Tq,Hq,D], lse [Hq,Tq],
    lse_excl [Hq,Tq]) in fp64. ``heads`` restricts the computation to some
    q-heads (other entries are left NaN)."""
    cu_q, cu_k, G = _check_problem(q, k, v, cu_q, cu_k, sinks)
    Tq, Hq, D = q.shape
    out = np.full((Tq, Hq, D), np.nan)
    lse = np.full((Hq, Tq), np.nan)
    lse_excl = np.full((Hq, Tq), np.nan)
    heads = range(Hq) if heads is None else heads
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        keep = keep_mask(q1 - q0, k1 - k0, causal, win_left, win_right)
        for h in heads:
            hk = h // G
            s = float(sinks[h])
            for r0, r1, j0, j1 in _row_blocks(keep, block_rows):
                f = _slice_forward(_f64(q[q0 + r0:q0 + r1, h]),
                                   _f64(k[k0 + j0:k0 + j1, hk]),
                                   _f64(v[k0 + j0:k0 + j1, hk]),
                                   s, scale, keep[r0:r1, j0:j1])
                out[q0 + r0:q0 + r1, h] = f["out"]
                lse[h, q0 + r0:q0 + r1] = f["lse"]
                lse_excl[h, q0 + r0:q0 + r1] = f["lse_excl"]
    return out, lse, lse_excl


def sink_attention_backward(dout, q, k, v, cu_q, cu_k, sinks, scale, causal,
                            win_left=-1, win_right=-1, block_rows=512,
                            heads=None):
    """Forward + backward over a packed batch, all fp64. Returns
    (dq [Tq,Hq,D], dk [Tk,Hk,D], dv [Tk,Hk,D], dsink [Hq]). dk/dv sum the
    contributions of the q-heads of each GQA group. With ``heads`` given,
    only those q-heads contribute (dk/dv then hold partial group sums and
    dq/dsink of other heads are NaN)."""
    cu_q, cu_k, G = _check_problem(q, k, v, cu_q, cu_k, sinks)
    Tq, Hq, D = q.shape
    Tk, Hk, _ = k.shape
    dq = np.full((Tq, Hq, D), np.nan)
    dk = np.zeros((Tk, Hk, D))
    dv = np.zeros((Tk, Hk, D))
    dsink = np.full(Hq, np.nan)
    heads = range(Hq) if heads is None else heads
    for h in heads:
        dsink[h] = 0.0
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        keep = keep_mask(q1 - q0, k1 - k0, causal, win_left, win_right)
        for h in heads:
            hk = h // G
            s = float(sinks[h])
            for r0, r1, j0, j1 in _row_blocks(keep, block_rows):
                Q = _f64(q[q0 + r0:q0 + r1, h])
                K = _f64(k[k0 + j0:k0 + j1, hk])
                V = _f64(v[k0 + j0:k0 + j1, hk])
                f = _slice_forward(Q, K, V, s, scale, keep[r0:r1, j0:j1])
                gq, gk, gv, gs = _slice_backward(
                    _f64(dout[q0 + r0:q0 + r1, h]), Q, K, V, f, scale)
                dq[q0 + r0:q0 + r1, h] = gq
                dk[k0 + j0:k0 + j1, hk] += gk
                dv[k0 + j0:k0 + j1, hk] += gv
                dsink[h] += gs
    return dq, dk, dv, dsink


def sink_attention_dsink(dout, q, k, v, cu_q, cu_k, sinks, scale, causal,
                         win_left=-1, win_right=-1, block_rows=512, heads=None):
    """Only the sink gradient, [Hq] (NaN for heads not computed): the
    forward per slice, then dsink_h = -sum_i p_sink,i (dO_i . out_i) -- the
    same sum _slice_backward forms, without the dq/dk/dv products."""
    cu_q, cu_k, G = _check_problem(q, k, v, cu_q, cu_k, sinks)
    Hq = q.shape[1]
    dsink = np.full(Hq, np.nan)
    heads = range(Hq) if heads is None else heads
    for h in heads:
        dsink[h] = 0.0
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        keep = keep_mask(q1 - q0, k1 - k0, causal, win_left, win_right)
        for h in heads:
            hk = h // G
            for r0, r1, j0, j1 in _row_blocks(keep, block_rows):
                f = _slice_forward(_f64(q[q0 + r0:q0 + r1, h]),
                                   _f64(k[k0 + j0:k0 + j1, hk]),
                                   _f64(v[k0 + j0:k0 + j1, hk]),
                                   float(sinks[h]), scale, keep[r0:r1, j0:j1])
                D = (_f64(dout[q0 + r0:q0 + r1, h]) * f["out"]).sum(axis=1)
                dsink[h] += float(-(f["p_sink"] * D).sum())
    return dsink


def sink_attention_rows(q, k, v, cu_q, cu_k, sinks, scale, causal,
                        win_left, win_right, rows, dout=None):
    """Forward (and, with ``dout``, the dq row) for sampled (token, q-head)
    pairs only: each row is independent of every other row, so a sample of
    a large problem is checked exactly. Returns a list of dicts with keys
    out [D], lse, and dq [D] when dout is given."""
    cu_q, cu_k, G = _check_problem(q, k, v, cu_q, cu_k, sinks)
    res = []
    for t, h in rows:
        b = int(np.searchsorted(cu_q, t, side="right") - 1)
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        i = t - q0
        keep = keep_row(i, q1 - q0, k1 - k0, causal, win_left, win_right)[None, :]
        hk = h // G
        Q = _f64(q[t:t + 1, h])
        K = _f64(k[k0:k1, hk])
        V = _f64(v[k0:k1, hk])
        f = _slice_forward(Q, K, V, float(sinks[h]), scale, keep)
        r = {"out": f["out"][0], "lse": float(f["lse"][0])}
        if dout is not None:
            gq, _, _, _ = _slice_backward(_f64(dout[t:t + 1, h]), Q, K, V, f,
                                          scale)
            r["dq"] = gq[0]
        res.append(r)
    return res


# ---------------------------------------------------------------------------
# softmax_n -- "Flash-Attention-Softmax-N (README)", introduction formula.
# ---------------------------------------------------------------------------
def sink_logit_for_n(n):
    """softmax_n adds n to the denominator: the same as a sink logit ln n
    (n = 0 gives -inf, i.e. the vanilla softmax)."""
    if n < 0:
        raise ValueError("softmax_n needs n >= 0")
    return NEG_INF if n == 0 else float(np.log(n))


def softmax_n(x, n, axis=-1):
    """exp(x_i) / (n + sum_j exp(x_j)), written out literally in fp64 with a
    max shift (the shift cancels; n is scaled by e^-max to match)."""
    x = _f64(x)
    mx = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - mx)
    return e / (n * np.exp(-mx) + e.sum(axis=axis, keepdims=True))


# ---------------------------------------------------------------------------
# Tile bookkeeping -- the work split that the CANN page's metadata call
# produces ("CANN flash_attn" Function: metadata records the task split),
# with inactive tiles skipped as in "hf-attention-normalizers", Packed
# Variable-Length Attention (one combined grid, inactive tiles masked).
# Brute force: every element of every tile is enumerated.
# ---------------------------------------------------------------------------
DEAD, PARTIAL, FULL = 0, 1, 2


def classify_tiles(len_q, len_k, tile_q, tile_k, causal, win_left, win_right):
    """[ceil(Lq/tile_q), ceil(Lk/tile_k)] array of DEAD / PARTIAL / FULL.
    DEAD: no kept element. FULL: every element inside the sequence bounds
    and kept. PARTIAL: anything else."""
    nq = -(-len_q // tile_q)
    nk = -(-len_k // tile_k)
    keep = keep_mask(len_q, len_k, causal, win_left, win_right)
    cls = np.zeros((nq, nk), dtype=np.int64)
    for a in range(nq):
        for c in range(nk):
            blk = keep[a * tile_q:(a + 1) * tile_q, c * tile_k:(c + 1) * tile_k]
            if not blk.any():
                cls[a, c] = DEAD
            elif blk.shape == (tile_q, tile_k) and blk.all():
                cls[a, c] = FULL
            else:
                cls[a, c] = PARTIAL
    return cls


def _span(flags):
    """(lo, hi) of the True entries of a 1-D array, asserted contiguous;
    (0, 0) when there are none."""
    idx = np.nonzero(flags)[0]
    if idx.size == 0:
        return 0, 0
    lo, hi = int(idx[0]), int(idx[-1]) + 1
    assert flags[lo:hi].all(), "live/full tiles must be contiguous"
    return lo, hi


def _full_span(live_lo, cls_line):
    lo, hi = _span(cls_line == FULL)
    if lo == hi:
        return live_lo, live_lo
    return lo, hi


def _dispatch_order(items):
    """Sequences by their total live tile count (descending, ties: lower b
    first); inside a sequence live tile count descending, then tile index."""
    work = {}
    for it in items:
        work[it[0]] = work.get(it[0], 0) + (it[3] - it[2])
    items.sort(key=lambda it: (-work[it[0]], it[0], -(it[3] - it[2]), it[1]))
    return items


def forward_items(cu_q, cu_k, tile_q, tile_k, causal, win_left, win_right):
    """One item per (sequence b, q tile qt), including items with no live key
    tile (their rows still produce out = 0, lse = sink). Item =
    (b, qt, kt_lo, kt_hi, kf_lo, kf_hi): live key tiles [kt_lo, kt_hi), of
    which [kf_lo, kf_hi) are FULL (empty full range = (kt_lo, kt_lo); empty
    live range = (0, 0)). Order: _dispatch_order."""
    items = []
    for b in range(len(cu_q) - 1):
        Lq, Lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        if Lq == 0:
            continue
        cls = classify_tiles(Lq, Lk, tile_q, tile_k, causal, win_left,
                             win_right)
        for qt in range(cls.shape[0]):
            lo, hi = _span(cls[qt] != DEAD) if cls.shape[1] else (0, 0)
            flo, fhi = _full_span(lo, cls[qt]) if cls.shape[1] else (0, 0)
            items.append((b, qt, lo, hi, flo, fhi))
    return _dispatch_order(items)


def backward_items(cu_q, cu_k, tile_q, tile_k, causal, win_left, win_right):
    """One item per (sequence b, key tile kt), including key tiles that no
    query sees (their dK, dV are still written as 0). Item =
    (b, kt, qt_lo, qt_hi, qf_lo, qf_hi) over q tiles of tile_q rows, same
    conventions and order as forward_items."""
    items = []
    for b in range(len(cu_q) - 1):
        Lq, Lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        if Lk == 0:
            continue
        cls = classify_tiles(Lq, Lk, tile_q, tile_k, causal, win_left,
                             win_right)
        for kt in range(cls.shape[1]):
            col = cls[:, kt]
            lo, hi = _span(col != DEAD) if cls.shape[0] else (0, 0)
            flo, fhi = _full_span(lo, col) if cls.shape[0] else (0, 0)
            items.append((b, kt, lo, hi, flo, fhi))
    return _dispatch_order(items)


def decode_items(cu_q, cu_k, tile_k, chunk_keys, causal, win_left, win_right,
                 tail_keys=None, tail_percent=0):
    """Split-KV work for short query groups: for each sequence, the span of
    keys kept by at least one of its rows, rounded out to tile_k tiles. The
    sequences are ordered by span length (descending, ties: lower b first);
    each span is cut into chunks of chunk_keys keys (clipped to the span),
    except that the sequences whose preceding spans (in that order) already
    make up at least (100 - tail_percent)% of the total span length are cut
    into chunks of tail_keys keys. Returns (items, per_seq): items =
    (b, split, k_lo, k_hi), each sequence's chunks together in key order;
    per_seq[b] = (first item index, number of splits). The cutting and the
    order are the scheduler's choices (they decide no value), written out
    here so that its table can be compared item for item."""
    spans = []
    for b in range(len(cu_q) - 1):
        Lq, Lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        start = stop = 0
        if Lq > 0 and Lk > 0:
            cols = keep_mask(Lq, Lk, causal, win_left, win_right).any(axis=0)
            lo, hi = _span(cols)
            if hi > lo:
                start = (lo // tile_k) * tile_k
                stop = min(Lk, -(-hi // tile_k) * tile_k)
        spans.append((start, stop))
    order = sorted(range(len(spans)), key=lambda b: (-(spans[b][1] - spans[b][0]), b))
    total = sum(stop - start for start, stop in spans)
    items, per_seq, before = [], [None] * len(spans), 0
    for b in order:
        start, stop = spans[b]
        step = chunk_keys
        if tail_keys is not None and before * 100 >= (100 - tail_percent) * total:
            step = tail_keys
        before += stop - start
        mine = [(b, s, a, min(stop, a + step)) for s, a in enumerate(range(start, stop, step))]
        per_seq[b] = (len(items), len(mine))
        items.extend(mine)
    return items, per_seq


def merge_partials(outs, lses, sinks):
    """Attention over the union of disjoint key parts from the parts' own
    sink-free results ("CANN ops-transformer: flash_attn", Note on
    softmax_lse, which ring attention merges by; the sink enters once, as in
    the Formula section): lse = ln(e^s + sum_p e^{lse_p}) and out =
    sum_p e^{lse_p - lse} out_p. outs [P, Tq, Hq, D], lses [P, Hq, Tq],
    sinks [Hq] (-inf: none). Returns (out [Tq, Hq, D], lse [Hq, Tq])."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    s = np.asarray(sinks, dtype=np.float64)[None, :, None]          # [1, Hq, 1]
    terms = np.concatenate([np.broadcast_to(s, (1,) + lses.shape[1:]), lses], axis=0)
    m = terms.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    total = np.exp(terms - m_safe).sum(axis=0)                     # [Hq, Tq]
    lse = np.where(total > 0, m_safe + np.log(np.where(total > 0, total, 1.0)), -np.inf)
    w = np.where(np.isfinite(lse)[None], np.exp(lses - np.where(np.isfinite(lse), lse, 0.0)[None]), 0.0)
    out = np.einsum("pht,pthd->thd", w, outs)
    return out, lse


def gather_paged(cache, block_table, seqused, block_size):
    """Keys (or values) of a paged cache as packed rows. "CANN ops-transformer:
    flash_attn", Paged Attention parameter group and the PA_BBND k/v layout
    (num_blocks, block_size, KV_N, D): row r of sequence b is slot
    r % block_size of page block_table[b, r // block_size], for r <
    seqused[b]. Returns (rows [sum(seqused), ...], cu_seqlens [B+1] int32)."""
    parts, cu = [], [0]
    for b, used in enumerate(np.asarray(seqused, dtype=np.int64)):
        pages = np.asarray(block_table[b][:(used + block_size - 1) // block_size])
        rows = np.asarray(cache)[pages].reshape((-1,) + np.asarray(cache).shape[2:])
        parts.append(rows[:used])
        cu.append(cu[-1] + int(used))
    shape = (0,) + np.asarray(cache).shape[2:]
    packed = np.concatenate(parts, axis=0) if parts else np.zeros(shape, np.asarray(cache).dtype)
    return packed, np.asarray(cu, dtype=np.int32)


def count_kept_pairs(cu_q, cu_k, causal, win_left, win_right):
    """Number of kept (row, key) pairs per head -- the FLOP-count basis."""
    total = 0
    for b in range(len(cu_q) - 1):
        Lq, Lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        total += int(keep_mask(Lq, Lk, causal, win_left, win_right).sum())
    return total
