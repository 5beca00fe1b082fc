"""The C ABI on the host (no GPU): exported symbols, argument checks and
error codes, and the tile schedule compared bit for bit with the oracle's
brute-force bookkeeping."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from softmax_sink_amd import binding as B
from softmax_sink_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "sink_attn.h")

# header word indices / tile shapes as laid out by the library
W_MODE, W_FWDBM, W_FWDBN, W_BWDBM, W_BWDBN, W_DECBN, W_DECCHUNK = 14, 15, 16, 17, 18, 19, 20
W_DECTAIL, W_DECTAILPCT = 48, 49      # split-KV chunk of the grid's last sequences, share cut so
ITEM = 16                             # words per work item
W_NFWD, W_FWDOFF, W_NBWD, W_BWDOFF, W_NDEC, W_DECOFF, W_DECSEQ, W_DECROWS = range(21, 29)


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_symbol(L):
    text = open(HDR).read()
    names = set(re.findall(r"\b(sink_attn_[a-z_]+)\s*\(", text))
    assert {"sink_attn_metadata", "sink_attn_fwd", "sink_attn_bwd",
            "sink_attn_metadata_paged", "sink_attn_fwd_paged",
            "sink_attn_metadata_padded", "sink_attn_fwd_padded", "sink_attn_bwd_padded",
            "sink_attn_status_string", "sink_attn_abi_version",
            "sink_attn_arm_timing"} <= names
    for n in names:
        assert hasattr(L, n), n
    version = re.search(r"#define SINK_ATTN_ABI_VERSION (\d+)", text).group(1)
    assert B.abi_version() == int(version)
    for s in range(6):
        assert isinstance(B.status_string(s), str)


def _meta(cu_q, cu_k, hq=4, hk=2, d=128, causal=True, wl=-1, wr=-1, dtype=B.BF16):
    p = B.make_problem(cu_q, cu_k, hq, hk, d, causal, wl, wr, dtype)
    return p, B.sink_attn_metadata(p, cu_q, cu_k)


def _items(meta, n_word, off_word, width=6):
    n, off = meta[n_word], meta[off_word]
    return [tuple(int(x) for x in meta[off + ITEM * i: off + ITEM * i + width]) for i in range(n)]


def _check_against_oracle(cu_q, cu_k, causal, wl, wr, hq=4, hk=2):
    cu_q = np.asarray(cu_q, np.int32)
    cu_k = np.asarray(cu_k, np.int32)
    p, (meta, fws, bws) = _meta(cu_q, cu_k, hq, hk, 128, causal, wl, wr)
    fbm, fbn, bbm, bbn = meta[W_FWDBM], meta[W_FWDBN], meta[W_BWDBM], meta[W_BWDBN]
    assert _items(meta, W_NFWD, W_FWDOFF) == O.forward_items(cu_q, cu_k, fbm, fbn, causal, wl, wr)
    assert _items(meta, W_NBWD, W_BWDOFF) == O.backward_items(cu_q, cu_k, bbm, bbn, causal, wl, wr)
    ditems, per_seq = O.decode_items(cu_q, cu_k, meta[W_DECBN], meta[W_DECCHUNK], causal, wl, wr,
                                     meta[W_DECTAIL], meta[W_DECTAILPCT])
    # every item carries its sequence's first rows and lengths (words 8-11)
    for n_word, off_word in ((W_NFWD, W_FWDOFF), (W_NBWD, W_BWDOFF), (W_NDEC, W_DECOFF)):
        for it in meta[meta[off_word]: meta[off_word] + ITEM * meta[n_word]].reshape(-1, ITEM):
            b = it[0]
            assert tuple(it[8:12]) == (cu_q[b], cu_q[b + 1] - cu_q[b], cu_k[b], cu_k[b + 1] - cu_k[b])
    # the forward's regions lie in the prefix it reads (header word 47):
    # the split-KV items and per-sequence table in decode mode, else the
    # per-query-tile items; the backward's items lie past it
    pre, nb = int(meta[B.META_FWD_WORDS]), len(cu_q) - 1
    if meta[W_MODE] == 1:
        assert meta[W_DECOFF] + ITEM * meta[W_NDEC] <= pre and meta[W_DECSEQ] + 2 * nb <= pre
        assert meta[W_FWDOFF] >= pre
    else:
        assert meta[W_FWDOFF] + ITEM * meta[W_NFWD] <= pre
    assert meta[W_BWDOFF] >= pre and pre <= len(meta)
    if meta[W_MODE] == 0:
        # prefill tables carry no split-KV items (the per-sequence table is
        # all zeros); compare the oracle's split items in decode mode only
        assert meta[W_NDEC] == 0 and meta[W_DECROWS] == 0
        seq = meta[meta[W_DECSEQ]: meta[W_DECSEQ] + 2 * (len(cu_q) - 1)]
        assert not seq.any()
        return meta
    assert _items(meta, W_NDEC, W_DECOFF, 4) == ditems
    seq = meta[meta[W_DECSEQ]: meta[W_DECSEQ] + 2 * (len(cu_q) - 1)].reshape(-1, 2)
    assert [tuple(int(x) for x in r) for r in seq] == per_seq
    # partial-row bases: running sum of (query rows x q-heads) over the items
    bases = [int(meta[meta[W_DECOFF] + ITEM * i + 4]) for i in range(meta[W_NDEC])]
    want, acc = [], 0
    for b, _, _, _ in ditems:
        want.append(acc)
        acc += int(cu_q[b + 1] - cu_q[b]) * hq
    assert bases == want and meta[W_DECROWS] == acc
    return meta


def test_schedule_matches_oracle_random():
    rng = np.random.default_rng(123)
    for trial in range(60):
        Bn = int(rng.integers(1, 6))
        lq = rng.integers(0, 300, Bn)
        lk = rng.integers(0, 300, Bn)
        if trial % 3 == 0:
            lk = lq.copy()
        lq[0] = max(1, lq[0]); lk[0] = max(1, lk[0])
        causal = bool(rng.integers(0, 2))
        wl = int(rng.choice([-1, 0, 1, 17, 64, 200]))
        wr = 0 if causal and rng.integers(0, 2) else (-1 if causal else int(rng.choice([-1, 0, 5, 100])))
        cu_q = np.r_[0, np.cumsum(lq)].astype(np.int32)
        cu_k = np.r_[0, np.cumsum(lk)].astype(np.int32)
        _check_against_oracle(cu_q, cu_k, causal, wl, wr)


@pytest.mark.parametrize("d", [128, 256])
def test_schedule_matches_oracle_at_tile_edges(d):
    """Lengths within two rows of a tile multiple and windows on either side
    of the tile widths, where the live and full tile spans change: the
    library's items (computed from the row bounds) against the oracle's
    element-by-element tile classes. D = 256 walks 32-row backward tiles."""
    rng = np.random.default_rng(77 + d)
    edges = [64 * m + e for m in range(1, 9) for e in (-2, -1, 0, 1, 2)]
    wins = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 300]
    for trial in range(40):
        Bn = int(rng.integers(1, 4))
        lq = rng.choice(edges, Bn)
        lk = lq.copy() if trial % 4 == 0 else rng.choice(edges, Bn)
        causal = bool(trial % 2)
        wl = int(rng.choice([-1] + wins))
        wr = (0 if rng.integers(0, 2) else -1) if causal else int(rng.choice([-1] + wins))
        cu_q = np.r_[0, np.cumsum(lq)].astype(np.int32)
        cu_k = np.r_[0, np.cumsum(lk)].astype(np.int32)
        p, (meta, _, _) = _meta(cu_q, cu_k, 4, 2, d, causal, wl, wr)
        fbm, fbn, bbm, bbn = meta[W_FWDBM], meta[W_FWDBN], meta[W_BWDBM], meta[W_BWDBN]
        assert bbm == (32 if d == 256 else 64)
        assert _items(meta, W_NFWD, W_FWDOFF) == O.forward_items(cu_q, cu_k, fbm, fbn, causal, wl, wr)
        assert _items(meta, W_NBWD, W_BWDOFF) == O.backward_items(cu_q, cu_k, bbm, bbn, causal, wl, wr)


def test_split_kv_schedule_matches_oracle_random():
    """Decode-mode tables (query rows x GQA group <= 64): split-KV items,
    per-sequence table and partial-row bases against the oracle."""
    rng = np.random.default_rng(321)
    n_decode = 0
    for trial in range(60):
        Bn = int(rng.integers(1, 7))
        lq = rng.integers(0, 33, Bn)
        lk = rng.integers(0, 5000, Bn)
        lq[0] = max(1, lq[0]); lk[0] = max(1, lk[0])
        causal = bool(rng.integers(0, 2))
        wl = int(rng.choice([-1, 0, 1, 17, 64, 2100]))
        wr = 0 if causal and rng.integers(0, 2) else (-1 if causal else int(rng.choice([-1, 0, 5, 100])))
        cu_q = np.r_[0, np.cumsum(lq)].astype(np.int32)
        cu_k = np.r_[0, np.cumsum(lk)].astype(np.int32)
        m = _check_against_oracle(cu_q, cu_k, causal, wl, wr, hq=4, hk=2)
        n_decode += int(m[W_MODE] == 1)
    assert n_decode == 60


def test_schedule_matches_oracle_on_workload_lengths():
    rng = np.random.default_rng(2)
    lens = rng.integers(64, 2049, 16)
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    m = _check_against_oracle(cu, cu, True, -1, -1, 32, 32)
    assert m[W_MODE] == 0
    cu4 = np.arange(0, 32769, 8192, dtype=np.int32)
    _check_against_oracle(cu4, cu4, True, 1024, 0, 64, 8)
    rng = np.random.default_rng(5)
    lq, lk = rng.integers(1, 17, 64), rng.integers(512, 32769, 64)
    m = _check_against_oracle(np.r_[0, np.cumsum(lq)].astype(np.int32),
                              np.r_[0, np.cumsum(lk)].astype(np.int32), True, -1, -1, 32, 8)
    assert m[W_MODE] == 1          # 16 rows x 4 heads fit one split-KV group


def test_metadata_two_call_protocol_and_sizes(L):
    cu = np.array([0, 100, 300], np.int32)
    p = B.make_problem(cu, cu, 8, 2, 128, True)
    words, fws, bws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st = L.sink_attn_metadata(ctypes.byref(p), B._i32p(cu), B._i32p(cu), None, 0,
                              ctypes.byref(words), ctypes.byref(fws), ctypes.byref(bws))
    assert st == B.OK and words.value > 48
    small = np.zeros(10, np.int32)
    st = L.sink_attn_metadata(ctypes.byref(p), B._i32p(cu), B._i32p(cu), B._i32p(small), 10,
                              ctypes.byref(words), ctypes.byref(fws), ctypes.byref(bws))
    assert st == B.E_BUFFER_TOO_SMALL
    meta, f, b = B.sink_attn_metadata(p, cu, cu)
    assert meta[0] == 0x4B4E4953 and meta[1] == B.abi_version() and len(meta) == words.value
    # bwd workspace: D [Hq,Tq] fp32 + per-block dsink partials (no dQ accumulator)
    assert 300 * 8 * 4 <= b < 300 * 8 * 4 + 4096
    assert f == 0       # prefill mode needs no forward scratch


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, B.E_INVALID), ("batch", 70000, B.E_INVALID),
    ("num_heads_q", 6, B.E_INVALID),           # not a multiple of num_heads_k = 4
    ("num_heads_k", 0, B.E_INVALID),
    ("head_dim", 96, B.E_UNSUPPORTED), ("dtype", 7, B.E_UNSUPPORTED),
    ("win_left", -2, B.E_INVALID), ("win_right", 3, B.E_INVALID),   # causal + right window
    ("causal", 2, B.E_INVALID), ("max_seqlen_q", 99, B.E_INVALID),
    ("max_seqlen_k", 201, B.E_INVALID), ("total_q", 299, B.E_INVALID),
    ("total_k", 0, B.E_INVALID),
])
def test_metadata_rejects(field, value, status):
    cu = np.array([0, 100, 300], np.int32)
    p = B.make_problem(cu, cu, 8, 4, 128, True)
    setattr(p, field, value)
    with pytest.raises(B.SinkAttnError) as e:
        B.sink_attn_metadata(p, cu, cu)
    assert e.value.status == status


def test_metadata_rejects_bad_cu_seqlens():
    p = B.make_problem([0, 5, 9], [0, 5, 9], 2, 2, 64, False)
    for cq in ([1, 5, 9], [0, 6, 5], [0, 5, 8]):
        with pytest.raises(B.SinkAttnError) as e:
            B.sink_attn_metadata(p, np.array(cq, np.int32), np.array([0, 5, 9], np.int32))
        assert e.value.status == B.E_INVALID


def test_zero_length_sequences_allowed():
    cu_q = np.array([0, 0, 7, 7, 12], np.int32)
    cu_k = np.array([0, 3, 3, 9, 20], np.int32)
    _check_against_oracle(cu_q, cu_k, True, -1, -1)
    _check_against_oracle(cu_q, cu_k, False, 2, 1)


FAKE = 0x10000  # an aligned, never-dereferenced address: every call below fails its checks first


def _fwd(p, meta, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, sinks=FAKE, scale=0.1,
                out=FAKE, lse=FAKE, workspace=None, workspace_bytes=0)
    args.update(kw)
    return B.sink_attn_fwd(p, meta, FAKE, args["q"], args["k"], args["v"], args["cu_q"],
                           args["cu_k"], args["sinks"], args["scale"], args["out"],
                           args["lse"], args["workspace"], args["workspace_bytes"],
                           stream=0, check=False)


def _bwd(p, meta, **kw):
    args = dict(dout=FAKE, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, cu_q=FAKE,
                cu_k=FAKE, sinks=FAKE, scale=0.1, dq=FAKE, dk=FAKE, dv=FAKE, dsink=FAKE,
                workspace=FAKE, workspace_bytes=1 << 40)
    args.update(kw)
    a = args
    return B.sink_attn_bwd(p, meta, FAKE, a["dout"], a["q"], a["k"], a["v"], a["out"],
                           a["lse"], a["cu_q"], a["cu_k"], a["sinks"], a["scale"], a["dq"],
                           a["dk"], a["dv"], a["dsink"], a["workspace"],
                           a["workspace_bytes"], stream=0, check=False)


def test_fwd_bwd_argument_checks():
    cu = np.array([0, 40, 100], np.int32)
    p, (meta, fws, bws) = _meta(cu, cu, 4, 2, 128, True)
    assert _fwd(p, meta, q=None) == B.E_INVALID
    assert _fwd(p, meta, lse=FAKE + 4) == B.E_INVALID          # misaligned
    assert _fwd(p, meta, scale=0.0) == B.E_INVALID
    assert _fwd(p, meta, scale=float("nan")) == B.E_INVALID
    assert _fwd(p, None) == B.E_INVALID
    other = B.make_problem(cu, cu, 4, 2, 128, False)
    assert _fwd(other, meta) == B.E_META_MISMATCH
    bad = meta.copy(); bad[0] ^= 1
    assert _fwd(p, bad) == B.E_META_MISMATCH
    assert _bwd(p, meta, dsink=None) == B.E_INVALID            # sink given, dsink missing
    assert _bwd(p, meta, sinks=None) == B.E_INVALID
    assert _bwd(p, meta, workspace_bytes=bws - 1) == B.E_BUFFER_TOO_SMALL
    assert _bwd(p, meta, dq=None) == B.E_INVALID
    assert _bwd(other, meta) == B.E_META_MISMATCH
    # decode-mode forward needs its split-KV scratch
    cq = np.array([0, 3, 5], np.int32); ck = np.array([0, 900, 3000], np.int32)
    p2, (meta2, fws2, _) = _meta(cq, ck, 8, 2, 128, True)
    assert meta2[W_MODE] == 1 and fws2 > 0
    assert _fwd(p2, meta2, workspace=FAKE, workspace_bytes=fws2 - 1) == B.E_BUFFER_TOO_SMALL
    assert _fwd(p2, meta2, workspace=None, workspace_bytes=fws2) == B.E_INVALID
    assert B.lib().sink_attn_arm_timing(FAKE, None) == B.E_INVALID
    assert B.lib().sink_attn_arm_timing(None, None) == B.OK


# ---------------------------------------------------------------------------
# paged K/V
# ---------------------------------------------------------------------------
W_PAGED = 36   # header words: paged flag, block size, table columns, pages, table hash


def _paged_case(bs=16, seed=3, lq=(1, 3, 2), lk=(40, 0, 100), hq=8, hk=2):
    rng = np.random.default_rng(seed)
    need = [(n + bs - 1) // bs for n in lk]
    table = np.zeros((len(lk), max(need) + 1), np.int32)
    perm = rng.permutation(sum(need) + 3).astype(np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    cu_q = np.r_[0, np.cumsum(lq)].astype(np.int32)
    used = np.asarray(lk, np.int32)
    kv = B.PagedKV(bs, table.shape[1], len(perm))
    p = B.make_problem_paged(cu_q, used, hq, hk, 128, True)
    return p, kv, cu_q, used, table


def test_paged_metadata_matches_oracle_schedule():
    for bs in (16, 48, 1024):
        p, kv, cu_q, used, table = _paged_case(bs)
        meta, fws = B.sink_attn_metadata_paged(p, kv, cu_q, used, table)
        assert fws > 0 and meta[W_MODE] == 1
        assert meta[W_PAGED:W_PAGED + 4].tolist() == [1, bs, table.shape[1], kv.num_blocks]
        cu_k = np.r_[0, np.cumsum(used)].astype(np.int32)
        ditems, per_seq = O.decode_items(cu_q, cu_k, meta[W_DECBN], meta[W_DECCHUNK], True, -1, -1,
                                         meta[W_DECTAIL], meta[W_DECTAILPCT])
        assert _items(meta, W_NDEC, W_DECOFF, 4) == ditems
        # a paged table serves the forward only: in decode mode it holds
        # neither backward nor per-query-tile items
        assert meta[W_NBWD] == 0 and meta[W_NFWD] == 0
        # the same problem through the contiguous call gives the same schedule
        meta_c, _, _ = B.sink_attn_metadata(p, cu_q, cu_k)
        assert meta_c[W_PAGED] == 0
        n = meta[W_NDEC]
        its = meta[meta[W_DECOFF]:meta[W_DECOFF] + ITEM * n].reshape(n, ITEM)
        its_c = meta_c[meta_c[W_DECOFF]:meta_c[W_DECOFF] + ITEM * n].reshape(n, ITEM)
        # identical but for the first key row (word 10): 0 in a paged cache
        assert np.array_equal(np.delete(its, 10, axis=1), np.delete(its_c, 10, axis=1))
        assert not its[:, 10].any() and np.array_equal(its_c[:, 10], cu_k[its_c[:, 0]])


def test_paged_metadata_rejects():
    p, kv, cu_q, used, table = _paged_case()
    def status(**kw):
        args = dict(p=p, kv=kv, cu_q=cu_q, used=used, table=table)
        args.update(kw)
        with pytest.raises(B.SinkAttnError) as e:
            B.sink_attn_metadata_paged(args["p"], args["kv"], args["cu_q"], args["used"],
                                       args["table"])
        return e.value.status
    for bs in (0, 8, 24, 2048):
        assert status(kv=B.PagedKV(bs, kv.max_blocks_per_seq, kv.num_blocks)) == B.E_INVALID
    assert status(kv=B.PagedKV(16, kv.max_blocks_per_seq, 0)) == B.E_INVALID
    assert status(kv=B.PagedKV(16, kv.max_blocks_per_seq, kv.num_blocks, 2)) == B.E_INVALID
    bad = table.copy(); bad[2, 0] = kv.num_blocks
    assert status(table=bad) == B.E_INVALID
    bad = table.copy(); bad[0, 0] = -1
    assert status(table=bad) == B.E_INVALID
    too_long = used.copy(); too_long[2] = 16 * kv.max_blocks_per_seq + 1
    p2 = B.make_problem_paged(cu_q, too_long, 8, 2, 128, True)
    assert status(p=p2, used=too_long) == B.E_INVALID
    wrong_total = B.make_problem_paged(cu_q, used, 8, 2, 128, True)
    wrong_total.total_k += 1
    assert status(p=wrong_total) == B.E_INVALID
    assert status(p=B.make_problem_paged(cu_q, used, 8, 2, 128, True, dtype=B.FP32)) == \
        B.E_UNSUPPORTED
    padded = B.make_problem_paged(cu_q, used, 8, 2, 128, True)
    padded.layout_q = padded.layout_out = B.BSND
    assert status(p=padded) == B.E_INVALID


def test_paged_long_queries_take_the_prefill_schedule():
    """40 query rows x 4 heads of a group exceed one split-KV group: the
    paged table then carries the tiled forward items of the same lengths."""
    p, kv, cu_q, used, table = _paged_case()
    long_q = np.array([0, 40, 41, 42], np.int32)
    pl = B.make_problem_paged(long_q, used, 8, 2, 128, True)
    meta, fws = B.sink_attn_metadata_paged(pl, kv, long_q, used, table)
    cu_k = np.r_[0, np.cumsum(used)].astype(np.int32)
    _, (mc, _, _) = _meta(long_q, cu_k, 8, 2, 128, True)
    assert meta[W_MODE] == 0 and mc[W_MODE] == 0 and fws == 0
    assert _items(meta, W_NFWD, W_FWDOFF) == _items(mc, W_NFWD, W_FWDOFF)
    assert meta[W_PAGED] == 1


def test_paged_entries_only_checked_where_used():
    # table entries past a sequence's last page are never read, so need not be valid
    p, kv, cu_q, used, table = _paged_case()
    table[:, -1] = 99999
    B.sink_attn_metadata_paged(p, kv, cu_q, used, table)


def test_paged_fwd_argument_checks():
    p, kv, cu_q, used, table = _paged_case()
    meta, fws = B.sink_attn_metadata_paged(p, kv, cu_q, used, table)
    cu_k = np.r_[0, np.cumsum(used)].astype(np.int32)
    meta_c, fws_c, bws_c = B.sink_attn_metadata(p, cu_q, cu_k)

    def fwdp(meta_host, kv_=kv, **kw):
        args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cu_q=FAKE, used=FAKE, sinks=FAKE,
                    out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40)
        args.update(kw)
        a = args
        return B.sink_attn_fwd_paged(p, kv_, meta_host, FAKE, a["q"], a["k"], a["v"], a["bt"],
                                     a["cu_q"], a["used"], a["sinks"], 0.1, a["out"],
                                     a["lse"], a["ws"], a["wsb"], stream=0, check=False)
    assert fwdp(meta_c) == B.E_META_MISMATCH                  # contiguous table
    assert fwdp(meta, kv_=B.PagedKV(32, kv.max_blocks_per_seq, kv.num_blocks)) == B.E_META_MISMATCH
    bnbd = B.PagedKV(kv.block_size, kv.max_blocks_per_seq, kv.num_blocks, B.PA_BNBD)
    assert fwdp(meta, kv_=bnbd) == B.E_META_MISMATCH       # the table was made for PA_BBND
    assert fwdp(meta, bt=None) == B.E_INVALID
    assert fwdp(meta, used=None) == B.E_INVALID
    assert fwdp(meta, wsb=fws - 1) == B.E_BUFFER_TOO_SMALL
    # a paged table is refused by the contiguous calls
    assert _fwd(p, meta, workspace=FAKE, workspace_bytes=1 << 40) == B.E_META_MISMATCH
    assert _bwd(p, meta) == B.E_META_MISMATCH


def test_merge_argument_checks():
    def m(parts=2, tq=10, hq=4, d=128, pd=B.BF16, od=B.BF16, po=FAKE, pl=FAKE, out=FAKE, lse=FAKE):
        return B.sink_attn_merge(parts, tq, hq, d, pd, od, po, pl, None, out, lse, stream=0,
                                 check=False)
    assert m(parts=0) == B.E_INVALID
    assert m(parts=4097) == B.E_INVALID
    assert m(tq=0) == B.E_INVALID
    assert m(hq=0) == B.E_INVALID
    assert m(d=96) == B.E_UNSUPPORTED
    assert m(pd=7) == B.E_UNSUPPORTED
    assert m(od=3) == B.E_UNSUPPORTED
    assert m(po=None) == B.E_INVALID
    assert m(lse=None) == B.E_INVALID
    assert m(out=FAKE + 8) == B.E_INVALID
    assert m(pl=FAKE + 2) == B.E_INVALID


def test_decode_workspace_sized_for_every_16bit_dtype():
    # the split-KV partials (fp32 O, m, l per (row, q-head, chunk)) must be
    # asked for whatever the 16-bit input type; the fp32 path has no split mode
    cq = np.array([0, 3, 5], np.int32)
    ck = np.array([0, 900, 3000], np.int32)
    sizes = {}
    for dt in (B.BF16, B.FP16, B.FP32):
        p = B.make_problem(cq, ck, 8, 2, 128, True, dtype=dt)
        meta, fws, _ = B.sink_attn_metadata(p, cq, ck)
        sizes[dt] = fws
        if dt != B.FP32:
            rows = meta[W_DECROWS]
            assert meta[W_MODE] == 1 and rows > 0 and fws >= rows * (128 + 2) * 4
    assert sizes[B.BF16] == sizes[B.FP16] and sizes[B.FP32] == 0
    # a paged fp16 table asks for the same
    p = B.make_problem_paged(cq, np.diff(ck), 8, 2, 128, True, dtype=B.FP16)
    table = np.arange(2 * 188, dtype=np.int32).reshape(2, 188)
    _, fws = B.sink_attn_metadata_paged(p, B.PagedKV(16, 188, 2 * 188), cq, np.diff(ck), table)
    assert fws == sizes[B.BF16]


# ---------------------------------------------------------------------------
# batch-padded layouts (BSND / BNSD, seqused)
# ---------------------------------------------------------------------------
W_LAYOUT = 41   # header words: layout_q, layout_out, seq_q, seq_k, seqused mask


def _padded(batch=3, sq=70, sk=130, uq=(70, 0, 33), uk=(130, 5, 64), layout="BSND",
            layout_out=None, causal=True, wl=-1, wr=-1, hq=8, hk=2):
    uq = None if uq is None else np.array(uq, np.int32)
    uk = None if uk is None else np.array(uk, np.int32)
    p = B.make_problem_padded(batch, sq, sk, uq, uk, hq, hk, 128, causal, wl, wr, B.BF16,
                              layout, layout_out)
    return p, uq, uk


@pytest.mark.parametrize("layout,lout", [("BSND", None), ("BNSD", None), ("BNSD", "BSND")])
def test_padded_schedule_equals_packed_schedule(layout, lout):
    """The work items depend on the sequence lengths only: a padded problem
    schedules exactly what the packed problem of its used lengths does."""
    for causal, wl, wr in ((True, -1, -1), (False, 17, 3), (False, -1, -1)):
        p, uq, uk = _padded(layout=layout, layout_out=lout, causal=causal, wl=wl, wr=wr)
        meta, fws, bws = B.sink_attn_metadata_padded(p, uq, uk)
        cu_q = np.r_[0, np.cumsum(uq)].astype(np.int32)
        cu_k = np.r_[0, np.cumsum(uk)].astype(np.int32)
        _, (pm, _, _) = _meta(cu_q, cu_k, 8, 2, 128, causal, wl, wr)
        for nw, ow, width in ((W_NFWD, W_FWDOFF, 6), (W_NBWD, W_BWDOFF, 6),
                              (W_NDEC, W_DECOFF, 5)):
            assert _items(meta, nw, ow, width) == _items(pm, nw, ow, width)
        assert meta[W_MODE] == pm[W_MODE]
        # padded rows: sequence b starts at row b * S (words 8 and 10)
        for nw, ow in ((W_NFWD, W_FWDOFF), (W_NBWD, W_BWDOFF), (W_NDEC, W_DECOFF)):
            for it in meta[meta[ow]: meta[ow] + ITEM * meta[nw]].reshape(-1, ITEM):
                assert tuple(it[8:12]) == (it[0] * 70, uq[it[0]], it[0] * 130, uk[it[0]])
        lay = B.LAYOUTS
        assert list(meta[W_LAYOUT:W_LAYOUT + 5]) == [lay[layout], lay[lout or layout], 70, 130, 3]
        # D [Hq, B*S_q] covers the padding rows too
        assert bws >= 8 * 3 * 70 * 4


def test_padded_without_seqused():
    p, _, _ = _padded(uq=None, uk=None)
    assert p.max_seqlen_q == 70 and p.max_seqlen_k == 130
    meta, _, _ = B.sink_attn_metadata_padded(p, None, None)
    assert meta[W_LAYOUT + 4] == 0
    cu_q = np.arange(4, dtype=np.int32) * 70
    cu_k = np.arange(4, dtype=np.int32) * 130
    _, (pm, _, _) = _meta(cu_q, cu_k, 8, 2, 128, True)
    assert _items(meta, W_NFWD, W_FWDOFF) == _items(pm, W_NFWD, W_FWDOFF)


def test_padded_metadata_rejects():
    p, uq, uk = _padded()

    def status(prob, a=uq, b=uk):
        with pytest.raises(B.SinkAttnError) as e:
            B.sink_attn_metadata_padded(prob, a, b)
        return e.value.status

    assert status(p, np.array([71, 0, 33], np.int32)) == B.E_INVALID    # used > S_q
    assert status(p, uq, np.array([130, -1, 64], np.int32)) == B.E_INVALID
    for field, value in (("total_q", 209), ("seq_k", 0), ("layout_out", 2), ("layout_q", 3),
                         ("max_seqlen_q", 69), ("max_seqlen_k", 131)):
        q, _, _ = _padded()
        setattr(q, field, value)
        assert status(q) == B.E_INVALID, field
    q, _, _ = _padded(layout="BNSD", layout_out="BSND")
    assert B.sink_attn_metadata_padded(q, uq, uk)[0][W_LAYOUT + 1] == B.BSND
    # a padded problem through the packed metadata call, and the reverse
    cu = np.array([0, 70, 140, 210], np.int32)
    with pytest.raises(B.SinkAttnError) as e:
        B.sink_attn_metadata(p, cu, cu)
    assert e.value.status == B.E_INVALID
    t = B.make_problem(cu, cu, 8, 2, 128, True)
    assert status(t, None, None) == B.E_INVALID
    t.seq_q = 70                     # TND with a padded row count
    with pytest.raises(B.SinkAttnError) as e:
        B.sink_attn_metadata(t, cu, cu)
    assert e.value.status == B.E_INVALID


def test_padded_fwd_bwd_argument_checks():
    p, uq, uk = _padded()
    meta, fws, bws = B.sink_attn_metadata_padded(p, uq, uk)

    def fwd(prob, m, used_q=FAKE, used_k=FAKE, **kw):
        a = dict(q=FAKE, out=FAKE)
        a.update(kw)
        return B.sink_attn_fwd_padded(prob, m, FAKE, a["q"], FAKE, FAKE, used_q, used_k, FAKE,
                                      0.1, a["out"], FAKE, FAKE, 1 << 40, stream=0,
                                      check=False)

    def bwd(prob, m, used_q=FAKE, used_k=FAKE, dsink=FAKE):
        return B.sink_attn_bwd_padded(prob, m, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      used_q, used_k, FAKE, 0.1, FAKE, FAKE, FAKE, dsink,
                                      FAKE, 1 << 40, stream=0, check=False)

    assert fwd(p, meta, q=None) == B.E_INVALID
    assert fwd(p, meta, out=FAKE + 2) == B.E_INVALID
    assert fwd(p, meta, used_q=None) == B.E_META_MISMATCH     # the table had seqused_q
    assert bwd(p, meta, used_k=None) == B.E_META_MISMATCH
    assert bwd(p, meta, dsink=None) == B.E_INVALID
    other, _, _ = _padded(layout="BNSD")
    assert fwd(other, meta) == B.E_META_MISMATCH               # layout differs
    # the packed calls refuse padded problems and tables, and the reverse
    assert _fwd(p, meta) == B.E_INVALID
    assert _bwd(p, meta) == B.E_INVALID
    cu = np.array([0, 40, 100], np.int32)
    t, (tmeta, _, _) = _meta(cu, cu, 8, 2, 128, True)
    assert fwd(t, tmeta, None, None) == B.E_INVALID
    assert bwd(t, tmeta, None, None) == B.E_INVALID


def test_head_dim_256_for_16_bit_types_only():
    cu = np.array([0, 100, 300], np.int32)
    for dt in (B.BF16, B.FP16):
        p = B.make_problem(cu, cu, 8, 2, 256, True, dtype=dt)
        meta, fws, bws = B.sink_attn_metadata(p, cu, cu)
        assert meta[5] == 256
        # the backward walks 32-row query tiles at this width; the items are
        # still the oracle's for the tile shape the header states
        assert meta[W_BWDBM] == 32 and meta[W_BWDBN] == 128
        assert _items(meta, W_NBWD, W_BWDOFF) == O.backward_items(cu, cu, 32, 128, True, -1, -1)
    for d, dt in ((256, B.FP32), (512, B.BF16), (192, B.BF16)):
        p = B.make_problem(cu, cu, 8, 2, d, True, dtype=dt)
        with pytest.raises(B.SinkAttnError) as e:
            B.sink_attn_metadata(p, cu, cu)
        assert e.value.status == B.E_UNSUPPORTED


def test_huge_windows_schedule_as_unbounded():
    """A window of max_seqlen_q + max_seqlen_k or more excludes no key: the
    schedule (and, in the GPU tests, every output) equals the unbounded one,
    also at the int32 limit, where the kernels' 32-bit mask arithmetic would
    otherwise wrap."""
    cu_q = np.array([0, 5, 300, 301], np.int32)
    cu_k = np.array([0, 200, 210, 600], np.int32)
    big = 2 ** 31 - 1
    for causal, wl, wr in ((True, big, 0), (False, big, big), (False, -1, big),
                           (False, 210 + 390, 600)):
        base_wl = -1 if wl >= 600 else wl
        base_wr = -1 if wr >= 600 else wr
        if causal:
            base_wr = wr
        m1 = _check_against_oracle(cu_q, cu_k, causal, wl, wr)
        m0 = _check_against_oracle(cu_q, cu_k, causal, base_wl, base_wr)
        for nw, ow in ((W_NFWD, W_FWDOFF), (W_NBWD, W_BWDOFF)):
            assert _items(m1, nw, ow) == _items(m0, nw, ow)


def test_problem_fields_must_fit_int32():
    cu = np.array([0, 10], np.int32)
    with pytest.raises(ValueError):
        B.make_problem(cu, cu, 4, 2, 128, False, 2 ** 32 + 5, -1)
    with pytest.raises(ValueError):
        B.make_problem(cu, cu, 4, 2, 128, False, -1, -2 ** 31 - 1)
    with pytest.raises(ValueError):
        B.make_problem_padded(2, 8, 8, None, None, 4, 2, 128, False, 2 ** 40, -1)
    p = B.make_problem(cu, cu, 4, 2, 128, False, 2 ** 31 - 1, 2 ** 31 - 1)
    assert p.win_left == 2 ** 31 - 1 and p.win_right == 2 ** 31 - 1


def test_noalloc_backward_rejects_problems_beyond_its_scratch(L):
    """sink_attn_bwd_noalloc refuses a problem whose backward scratch exceeds
    its static array (checked on the host before any device work; the
    device pointers here are never touched)."""
    tq = (B.NOALLOC_SCRATCH_BYTES // 4) // 32 + 64          # D alone overflows
    cu = np.array([0, tq], np.int32)
    p = B.make_problem(cu, cu, 32, 32, 128, True)
    meta, fws, bws = B.sink_attn_metadata(p, cu, cu)
    assert bws > B.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20                                            # 16-byte aligned, never read
    st = B.sink_attn_bwd_noalloc(p, meta, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                 fake, 0.1, fake, fake, fake, fake, stream=0, check=False)
    assert st == B.E_BUFFER_TOO_SMALL


@pytest.mark.parametrize("name,lens_q,lens_k,hk,chunk,tail", [
    # 64 sequences (the decode workload): 2312 blocks at 4096 keys, two
    # rounds and more, so the last 10% of the span length goes in 1024s
    ("decode_softmax_n", None, None, 8, 4096, 1024),
    # one 32k sequence: 64 blocks at 4096 keys; halved to 512 keys (512
    # blocks, one per slot); one round, no tail cut
    ("b1_k32k", [1], [32768], 8, 512, 512),
    # 16 x 16k: 512 blocks already at 4096 keys; one round, no tail cut
    ("b16_k16k", [2] * 16, [16384] * 16, 8, 4096, 4096),
    # a single short sequence stops at the shortest chunk
    ("b1_k1000", [3], [1000], 1, 512, 512),
])
def test_split_kv_chunk_choice(name, lens_q, lens_k, hk, chunk, tail):
    """The split-KV chunk is 4096 keys, halved down to 512 while the grid
    (items x kv-heads) has fewer than 512 blocks; when the grid has at least
    1024 blocks, the sequences in the last 10% of the span length (longest
    first) are cut into 1024-key items. The items equal the oracle's
    bookkeeping for those parameters."""
    if lens_q is None:
        lens_q, lens_k = W.decode_lengths()
        hq = 32
        cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    else:
        cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
        hq = 4 * hk
    _, (meta, _, _) = _meta(cu_q, cu_k, hq, hk, 128, True)
    assert meta[W_MODE] == 1
    assert (meta[W_DECCHUNK], meta[W_DECTAIL], meta[W_DECTAILPCT]) == (chunk, tail, 10)
    ditems, per_seq = O.decode_items(cu_q, cu_k, meta[W_DECBN], chunk, True, -1, -1, tail, 10)
    assert _items(meta, W_NDEC, W_DECOFF, 4) == ditems
    blocks = len(ditems) * hk
    assert blocks >= 512 or chunk == 512


def test_metadata_calls_from_many_host_threads_agree():
    """Calls are reentrant: eight host threads building tables for different
    problems at once (ctypes drops the GIL around the foreign call, so the
    C code runs concurrently) get exactly the tables of one-at-a-time calls."""
    import concurrent.futures as cf
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(48):
        n = int(rng.integers(1, 20))
        lq = rng.integers(0, 700, n)
        lk = lq + rng.integers(0, 300, n)
        lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        hk = int(rng.choice([1, 2, 8]))
        causal = bool(rng.integers(0, 2))
        wl = int(rng.choice([-1, 64, 500]))
        cases.append((cu_q, cu_k, 8, hk, 128, causal, wl, 0 if causal else -1))

    def table(c):
        cu_q, cu_k, hq, hk, d, causal, wl, wr = c
        return _meta(cu_q, cu_k, hq, hk, d, causal, wl, wr)[1]

    want = [table(c) for c in cases]
    for _ in range(3):
        with cf.ThreadPoolExecutor(8) as ex:
            got = list(ex.map(table, cases))
        for (m0, f0, b0), (m1, f1, b1) in zip(want, got):
            assert np.array_equal(m0, m1) and (f0, b0) == (f1, b1)
