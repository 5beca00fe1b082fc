"""Seeded synthetic inputs for sink attention (shared by tests and bench).

This module only draws numbers and lays them out; it holds none of the
attention arithmetic. Both the HIP path and the CPU oracle consume what it
produces, so it imports neither of them.

Recipe (one numpy ``default_rng(seed)`` stream per problem; draw order:
sequence lengths, q, k, v, dO, sinks):

* values are drawn as fp32 N(0, 1); for bf16 (fp16) problems they are
  rounded to bf16 (fp16) with round-to-nearest-even and kept as raw 16-bit
  patterns (``uint16``); ``as_f32`` widens them exactly;
* the softmax scale is the fp32 value of 1/sqrt(head_dim) unless given;
* sink logits are fp32: drawn N(0, 1) per q-head ("learnable offset"), or a
  constant ln n for softmax_n problems.

Five named configurations are the reference workloads:
``softmax1_fp32`` (1 x 128 x 128, 1 head, D 64, n = 1, non-causal),
``prefill_varlen`` (16 sequences, lengths uniform in [64, 2048], 32/32
heads, D 128, causal), ``train_varlen`` (8 sequences summing to 32768
tokens, lengths uniform in [1024, 8192], 32/32 heads, D 128, causal,
forward + backward), ``gqa_window`` (4 x 8192, 64/8 heads, D 128, causal
with window (1024, 0), forward + backward) and ``decode_softmax_n`` (64
sequences, q length uniform in [1, 16], kv length uniform in [512, 32768],
32/8 heads, D 128, bottom-right causal, n = 0.5), plus ``decode_paged``:
the same draw with its keys and values scattered into 16-row pages of a
paged cache in random page order (``paged_layout``, ``scatter_to_pages``),
``prefill_paged``: the ``prefill_varlen`` draw with its keys and values in
16-row pages (a prefill against a paged cache), ``gqa_window_bnsd``: the
``gqa_window`` draw laid out as BNSD
(``pad_rows``), and ``train_varlen_d256``: the ``train_varlen`` lengths with
16/16 heads of head_dim 256.
"""

import math
from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 24


def round_to_bf16_bits(x):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even.
    Inputs are finite normal draws (no NaN handling needed)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                       # finite inputs: no wrap-around
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, n, bf16, fp16=False):
    """n draws of N(0,1) in fp32, drawn chunk by chunk (same stream as one
    call), optionally rounded to bf16 or fp16 bits."""
    out = np.empty(n, dtype=np.uint16 if (bf16 or fp16) else np.float32)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        x = rng.standard_normal(b - a, dtype=np.float32)
        if fp16:
            out[a:b] = x.astype(np.float16).view(np.uint16)     # IEEE round to nearest even
        else:
            out[a:b] = round_to_bf16_bits(x) if bf16 else x
    return out


@dataclass
class Problem:
    name: str
    dtype: str                     # "bf16", "fp16" or "fp32"
    cu_q: np.ndarray               # int32 [B+1]
    cu_k: np.ndarray               # int32 [B+1]
    num_heads_q: int
    num_heads_k: int
    head_dim: int
    causal: bool
    win_left: int
    win_right: int
    scale: np.float32
    sinks: np.ndarray              # fp32 [Hq]; -inf allowed (no sink)
    q: np.ndarray                  # uint16 bf16 bits or fp32, [Tq,Hq,D]
    k: np.ndarray                  # [Tk,Hk,D]
    v: np.ndarray                  # [Tk,Hk,D]
    dout: np.ndarray               # [Tq,Hq,D]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.cu_q) - 1

    @property
    def total_q(self):
        return int(self.cu_q[-1])

    @property
    def total_k(self):
        return int(self.cu_k[-1])

    @property
    def max_seqlen_q(self):
        return int(np.diff(self.cu_q).max()) if self.batch else 0

    @property
    def max_seqlen_k(self):
        return int(np.diff(self.cu_k).max()) if self.batch else 0

    def as_f32(self, name):
        """Exact fp32 view of one of q, k, v, dout."""
        x = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(x)
        if self.dtype == "fp16":
            return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float32)
        return x

    def sub_batch(self, seqs):
        """A new Problem holding only the listed sequences (same heads,
        sinks, scale and mask) -- used to check samples of a large batch."""
        qs, ks, cq, ck = [], [], [0], [0]
        for b in seqs:
            qs.append(slice(int(self.cu_q[b]), int(self.cu_q[b + 1])))
            ks.append(slice(int(self.cu_k[b]), int(self.cu_k[b + 1])))
            cq.append(cq[-1] + qs[-1].stop - qs[-1].start)
            ck.append(ck[-1] + ks[-1].stop - ks[-1].start)
        cat = lambda x, sl: np.concatenate([x[s] for s in sl], axis=0)
        return Problem(self.name + "[sub]", self.dtype,
                       np.array(cq, np.int32), np.array(ck, np.int32),
                       self.num_heads_q, self.num_heads_k, self.head_dim,
                       self.causal, self.win_left, self.win_right, self.scale,
                       self.sinks, cat(self.q, qs), cat(self.k, ks),
                       cat(self.v, ks), cat(self.dout, qs), self.seed,
                       dict(self.meta, parent_seqs=list(seqs)))


def make_problem(seed, lens_q, lens_k, num_heads_q, num_heads_k, head_dim,
                 dtype="bf16", causal=True, win_left=-1, win_right=-1,
                 sinks="normal", scale=None, name="custom", rng=None):
    """Draw q, k, v, dO (and sinks) for given sequence lengths.

    sinks: "normal" (N(0,1) fp32 per q-head), a float (same logit for every
    head; -inf = no sink), or an explicit array of Hq fp32 values."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    bf16, fp16 = dtype == "bf16", dtype == "fp16"
    q = _normal(rng, Tq * num_heads_q * head_dim, bf16, fp16).reshape(Tq, num_heads_q, head_dim)
    k = _normal(rng, Tk * num_heads_k * head_dim, bf16, fp16).reshape(Tk, num_heads_k, head_dim)
    v = _normal(rng, Tk * num_heads_k * head_dim, bf16, fp16).reshape(Tk, num_heads_k, head_dim)
    dout = _normal(rng, Tq * num_heads_q * head_dim, bf16, fp16).reshape(Tq, num_heads_q,
                                                                        head_dim)
    if isinstance(sinks, str) and sinks == "normal":
        s = rng.standard_normal(num_heads_q, dtype=np.float32)
    elif np.isscalar(sinks):
        s = np.full(num_heads_q, sinks, dtype=np.float32)
    else:
        s = np.asarray(sinks, dtype=np.float32)
    if scale is None:
        scale = np.float32(1.0 / math.sqrt(head_dim))
    return Problem(name, dtype, cu_q, cu_k, num_heads_q, num_heads_k, head_dim,
                   bool(causal), int(win_left), int(win_right),
                   np.float32(scale), s, q, k, v, dout, seed)


@dataclass
class PagedLayout:
    """Where the key rows of each sequence live in a paged cache."""
    block_size: int
    block_table: np.ndarray        # int32 [B, max_blocks_per_seq]
    seqused: np.ndarray            # int32 [B], key rows per sequence
    num_blocks: int


def paged_layout(cu_k, block_size, seed, spare=0):
    """Sequence b gets ceil(L_b / block_size) distinct pages, taken in order
    from one random permutation of all num_blocks pages (no page shared);
    unused table entries are 0. `spare` extra pages stay unused."""
    lens = np.diff(np.asarray(cu_k, dtype=np.int64))
    need = (lens + block_size - 1) // block_size
    num_blocks = int(need.sum()) + int(spare)
    perm = np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)
    table = np.zeros((len(lens), max(1, int(need.max()) if len(need) else 1)), np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += int(n)
    return PagedLayout(int(block_size), table, lens.astype(np.int32), num_blocks)


def scatter_to_pages(x, cu_k, layout, cache_layout="BBND"):
    """Packed rows x [Tk, Hk, D] -> cache [num_blocks, block_size, Hk, D]
    (BBND; BNBD: [num_blocks, Hk, block_size, D]) with row r of sequence b
    in slot r % block_size of page block_table[b, r // block_size]; slots no
    row maps to are 0."""
    bs = layout.block_size
    cache = np.zeros((layout.num_blocks, bs) + x.shape[1:], dtype=x.dtype)
    for b in range(len(cu_k) - 1):
        rows = x[int(cu_k[b]):int(cu_k[b + 1])]
        for pg in range((len(rows) + bs - 1) // bs):
            chunk = rows[pg * bs:(pg + 1) * bs]
            cache[layout.block_table[b, pg], :len(chunk)] = chunk
    if cache_layout == "BNBD":
        return np.ascontiguousarray(cache.transpose(0, 2, 1, 3))
    if cache_layout != "BBND":
        raise ValueError(cache_layout)
    return cache


# Raw NaN patterns by element type: padding rows of the batch-padded layouts
# are filled with NaN so that any read of them shows in the results.
NAN_BITS = {"bf16": np.uint16(0x7FC0), "fp16": np.uint16(0x7E00), "fp32": np.float32(np.nan)}


def pad_rows(x, cu, seq, layout, fill):
    """Packed rows x [T, N, D] of sequences cu -> a batch-padded tensor with
    seq rows per sequence: "BSND" [B, seq, N, D] or "BNSD" [B, N, seq, D].
    Row i of sequence b lands at [b, i] (BSND) or [b, :, i] (BNSD); rows past
    a sequence's length hold `fill`."""
    nb = len(cu) - 1
    n, d = x.shape[1], x.shape[2]
    out = np.full((nb, seq, n, d), fill, dtype=x.dtype)
    for b in range(nb):
        rows = x[int(cu[b]):int(cu[b + 1])]
        out[b, :len(rows)] = rows
    if layout == "BNSD":
        out = np.ascontiguousarray(out.transpose(0, 2, 1, 3))
    elif layout != "BSND":
        raise ValueError(layout)
    return out


def _train_lengths(rng, n=8, total=32768, lo=1024, hi=8192):
    """n lengths uniform in [lo, hi] summing to total: draw n-1, set the last
    to the remainder, redraw all until the last is in range."""
    while True:
        head = rng.integers(lo, hi + 1, n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]])


def merge_inputs(seed, parts, total_q, num_heads_q, head_dim):
    """Synthetic sink-free partials for a context-parallel merge: partial
    outputs N(0, 1) as bf16 bits [parts, Tq, Hq, D], partial lse N(2, 3^2)
    fp32 [parts, Hq, Tq] (about one part in eight empty: -inf), sinks N(0, 1)
    fp32 [Hq]."""
    rng = np.random.default_rng(seed)
    outs = _normal(rng, parts * total_q * num_heads_q * head_dim, True).reshape(
        parts, total_q, num_heads_q, head_dim)
    lses = (rng.standard_normal((parts, num_heads_q, total_q), dtype=np.float32) * 3 + 2)
    lses[rng.random(lses.shape) < 0.125] = -np.inf
    sinks = rng.standard_normal(num_heads_q, dtype=np.float32)
    return outs, lses.astype(np.float32), sinks


CONFIG_NAMES = ("softmax1_fp32", "prefill_varlen", "train_varlen",
                "gqa_window", "decode_softmax_n")
DECODE_PAGE_ROWS = 16      # block size of the paged decode workload
DECODE_PAGE_SEED = 55


def _decode_draw():
    rng = np.random.default_rng(5)
    lq = rng.integers(1, 17, 64)
    lk = rng.integers(512, 32769, 64)
    return rng, lq, lk


def decode_lengths():
    """Query and key lengths of the decode workload (no tensors drawn)."""
    _, lq, lk = _decode_draw()
    return lq, lk


def config(name):
    """The named workload with its fixed seed."""
    if name == "softmax1_fp32":
        return make_problem(1, [128], [128], 1, 1, 64, dtype="fp32",
                            causal=False, sinks=0.0,
                            scale=np.float32(0.125), name=name)
    if name in ("prefill_varlen", "prefill_paged"):
        rng = np.random.default_rng(2)
        lens = rng.integers(64, 2049, 16)
        p = make_problem(2, lens, lens, 32, 32, 128, causal=True,
                         name=name, rng=rng)
        if name == "prefill_paged":
            p.meta["paged"] = paged_layout(p.cu_k, DECODE_PAGE_ROWS, DECODE_PAGE_SEED)
        return p
    if name == "train_varlen":
        rng = np.random.default_rng(3)
        lens = _train_lengths(rng)
        return make_problem(3, lens, lens, 32, 32, 128, causal=True,
                            name=name, rng=rng)
    if name == "train_varlen_d256":
        # the training lengths at head_dim 256 with half the heads (the same
        # FLOPs per kept pair and head-row bytes as train_varlen)
        rng = np.random.default_rng(3)
        lens = _train_lengths(rng)
        return make_problem(3, lens, lens, 16, 16, 256, causal=True,
                            name=name, rng=rng)
    if name == "gqa_window":
        lens = np.full(4, 8192)
        return make_problem(4, lens, lens, 64, 8, 128, causal=True,
                            win_left=1024, win_right=0, name=name)
    if name == "gqa_window_bnsd":
        # the same draw, handed over in the batch-padded BNSD layout (every
        # sequence is 8192 rows, so no row is padding)
        p = config("gqa_window")
        p.name = name
        p.meta["layout"] = "BNSD"
        return p
    if name in ("decode_softmax_n", "decode_paged"):
        rng, lq, lk = _decode_draw()
        p = make_problem(5, lq, lk, 32, 8, 128, causal=True,
                         sinks=np.float32(math.log(0.5)), name=name,
                         rng=rng)
        if name == "decode_paged":
            p.meta["paged"] = paged_layout(p.cu_k, DECODE_PAGE_ROWS, DECODE_PAGE_SEED)
        return p
    raise KeyError(name)
