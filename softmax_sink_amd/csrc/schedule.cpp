// Host-side problem checks and the varlen tile schedule (integer only).
//
// The schedule follows the two-phase model of the "CANN ops-transformer:
// flash_attn" page (Function section: a metadata call records the task
// split, the main call consumes it) and the packed-varlen grid of the
// "hf-attention-normalizers" description (Packed Variable-Length Attention:
// one combined grid over the packed batch, inactive tiles skipped). The mask
// is the bottom-right aligned causal/window mask of "pytorch/pytorch issue
// #108108" (Proposal section) with inclusive (left, right) windows.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <utility>
#include <vector>

#include "sink_attn_internal.h"

namespace sinkattn {
namespace {

constexpr int64_t kInf = std::numeric_limits<int64_t>::max() / 4;

// Kept key interval of query row i is [lo(i), hi(i)] (before clipping to
// [0, Lk-1]); both ends are non-decreasing in i.
struct RowBounds {
  int64_t off;      // Lk - Lq
  int64_t wl;       // -1 = unbounded
  int64_t wr_eff;   // right reach past the diagonal, or kInf when unbounded
  int64_t lo(int64_t i) const { return wl >= 0 ? i + off - wl : -kInf; }
  int64_t hi(int64_t i) const { return wr_eff >= kInf ? kInf : i + off + wr_eff; }
};

RowBounds row_bounds(const sink_attn_problem& p, int64_t lq, int64_t lk) {
  RowBounds r;
  r.off = lk - lq;
  r.wl = p.win_left;
  if (p.causal) r.wr_eff = 0;                  // causal requires win_right <= 0
  else r.wr_eff = p.win_right >= 0 ? p.win_right : kInf;
  return r;
}

// Tile spans of one work item in O(1). A tile is live when some row of it
// keeps some key of it, and full when it has its nominal shape and every
// row keeps every key. The kept keys of row i, [lo(i), hi(i)], move up by
// one key per row and are never empty (hi - lo = wl + wr_eff >= 0), so any
// run of rows keeps one contiguous key interval; the live tiles are those
// that interval meets, and the full tiles a contiguous run inside them.
// Spans are [lo, hi) with the canonical empty forms: no live tile ->
// (0, 0, 0, 0); no full tile -> full = (lo, lo).
void put_spans(int64_t lo, int64_t hi, int64_t flo, int64_t fhi, int32_t* out4) {
  if (hi <= lo) lo = hi = 0;
  if (fhi <= flo) flo = fhi = lo;
  out4[0] = static_cast<int32_t>(lo);
  out4[1] = static_cast<int32_t>(hi);
  out4[2] = static_cast<int32_t>(flo);
  out4[3] = static_cast<int32_t>(fhi);
}

// Key tiles of width bn over [0, lk) for the query rows [r0, r1).
void key_tile_spans(const RowBounds& rb, int64_t r0, int64_t r1, int64_t lk, int64_t bm,
                    int64_t bn, int32_t* out4) {
  const int64_t k0 = std::max<int64_t>(0, rb.lo(r0));
  const int64_t k1 = std::min<int64_t>(lk - 1, rb.hi(r1 - 1));   // kept keys [k0, k1]
  if (r1 <= r0 || k1 < k0) return put_spans(0, 0, 0, 0, out4);
  int64_t flo = 0, fhi = 0;
  if (r1 - r0 == bm) {
    // c0 >= lo(r1 - 1), c0 + bn - 1 <= hi(r0), c0 + bn <= lk
    const int64_t c_min = std::max<int64_t>(0, rb.lo(r1 - 1));
    const int64_t c_max = std::min<int64_t>(rb.hi(r0) - bn + 1, lk - bn);
    if (c_max >= c_min) {
      flo = (c_min + bn - 1) / bn;
      fhi = c_max / bn + 1;
    }
  }
  put_spans(k0 / bn, k1 / bn + 1, flo, fhi, out4);
}

// Query tiles of height bm over [0, lq) for the keys [c0, c1).
void query_tile_spans(const RowBounds& rb, int64_t c0, int64_t c1, int64_t lq, int64_t bm,
                      int64_t bn, int32_t* out4) {
  // rows with lo(i) <= c1 - 1 and hi(i) >= c0: [i0, i1)
  const int64_t i1 = rb.wl >= 0 ? std::min<int64_t>(lq, c1 - rb.off + rb.wl) : lq;
  const int64_t i0 = rb.wr_eff < kInf ? std::max<int64_t>(0, c0 - rb.off - rb.wr_eff) : 0;
  if (c1 <= c0 || i1 <= i0) return put_spans(0, 0, 0, 0, out4);
  int64_t flo = 0, fhi = 0;
  if (c1 - c0 == bn) {
    // r0 + bm <= lq, lo(r0 + bm - 1) <= c0, hi(r0) >= c1 - 1
    const int64_t r_top = (rb.wl >= 0 ? std::min<int64_t>(lq, c0 - rb.off + rb.wl + 1) : lq) - bm;
    const int64_t r_min = rb.wr_eff < kInf ? std::max<int64_t>(0, c1 - 1 - rb.off - rb.wr_eff) : 0;
    if (r_top >= r_min) {
      flo = (r_min + bm - 1) / bm;
      fhi = r_top / bm + 1;
    }
  }
  put_spans(i0 / bm, (i1 - 1) / bm + 1, flo, fhi, out4);
}

struct Item {
  int32_t w[kItemWords];
};

// Dispatch order: sequences by their total live tile count, descending
// (ties: lower index first); inside a sequence, live tile count descending,
// then tile index. Heavy work starts first, and the blocks that run at the
// same time mostly belong to one sequence, so they share its K/V (forward)
// or Q/dO (backward) tiles in L2.
// The items arrive grouped by sequence, each group in tile order, so the
// sequences are ordered once and each group is stably ordered by its live
// tile counts (linear when they are all equal, as in decode batches).
void sort_items(std::vector<Item>& v, int batch) {
  std::vector<int64_t> work(static_cast<size_t>(batch), 0);
  std::vector<size_t> first(static_cast<size_t>(batch) + 1, 0);
  for (const Item& it : v) {
    work[it.w[0]] += it.w[3] - it.w[2];
    ++first[static_cast<size_t>(it.w[0]) + 1];
  }
  for (int b = 0; b < batch; ++b) first[b + 1] += first[b];
  std::vector<int> order(static_cast<size_t>(batch));
  for (int b = 0; b < batch; ++b) order[b] = b;
  std::sort(order.begin(), order.end(), [&](int x, int y) {
    return work[x] != work[y] ? work[x] > work[y] : x < y;
  });
  // each group is ordered through (live count, position) keys, so that the
  // 64-byte items move once
  std::vector<Item> out;
  out.reserve(v.size());
  std::vector<std::pair<int32_t, uint32_t>> key;
  for (int b : order) {
    const size_t lo = first[b], hi = first[b + 1];
    bool sorted = true;
    for (size_t i = lo + 1; i < hi && sorted; ++i)
      sorted = v[i - 1].w[3] - v[i - 1].w[2] >= v[i].w[3] - v[i].w[2];
    if (sorted) {
      out.insert(out.end(), v.begin() + lo, v.begin() + hi);
      continue;
    }
    key.clear();
    for (size_t i = lo; i < hi; ++i)
      key.emplace_back(-(v[i].w[3] - v[i].w[2]), static_cast<uint32_t>(i));
    std::sort(key.begin(), key.end());       // count descending, then position
    for (const auto& k : key) out.push_back(v[k.second]);
  }
  v.swap(out);
}

// Split-KV blocks (items x kv-heads) of the spans cut into `chunk`-key pieces.
int64_t decode_blocks(const std::vector<int64_t>& span, int batch, int hk, int32_t chunk) {
  int64_t blocks = 0;
  for (int b = 0; b < batch; ++b) blocks += (span[2 * b + 1] - span[2 * b] + chunk - 1) / chunk * hk;
  return blocks;
}

// Key chunk of the split-KV items: kDecChunk, halved (down to kDecMinChunk)
// while the grid would have fewer than kDecMinBlocks blocks, so that short
// batches still fill the chip.
int32_t decode_chunk(const std::vector<int64_t>& span, int batch, int hk) {
  int32_t chunk = kDecChunk;
  for (;;) {
    const int64_t blocks = decode_blocks(span, batch, hk, chunk);
    if (blocks == 0 || blocks >= kDecMinBlocks || chunk / 2 < kDecMinChunk) return chunk;
    chunk /= 2;
  }
}

// Chunk of the sequences at the end of the grid: kDecTailChunk when the grid
// takes at least two rounds of kDecMinBlocks blocks (short blocks at the end
// then shorten the last round), else the chunk itself.
int32_t decode_tail_chunk(const std::vector<int64_t>& span, int batch, int hk, int32_t chunk) {
  return decode_blocks(span, batch, hk, chunk) >= 2 * kDecMinBlocks
             ? std::min<int32_t>(chunk, kDecTailChunk) : chunk;
}

// Split-KV items in dispatch order: sequences by their span length
// (descending, ties by b), each sequence's chunks contiguous and in key
// order (the combine finds chunk s of sequence b at item first(b) + s).
// Spans are cut into `chunk`-key pieces; the sequences that start in the
// last kDecTailPercent of the total span length (in that order) are cut into
// pieces of at most kDecTailChunk keys, so that the end of the grid is made
// of short blocks. Partial rows are numbered in item order; returns their
// count.
int64_t decode_items(const std::vector<int64_t>& span, int32_t chunk, int32_t tail_chunk,
                     int batch, const int32_t* cu_q, int hq, std::vector<Item>& dec,
                     std::vector<int32_t>& dec_seq) {
  std::vector<int> order(static_cast<size_t>(batch));
  int64_t total = 0;
  for (int b = 0; b < batch; ++b) {
    order[b] = b;
    total += span[2 * b + 1] - span[2 * b];
  }
  std::sort(order.begin(), order.end(), [&](int x, int y) {
    const int64_t wx = span[2 * x + 1] - span[2 * x], wy = span[2 * y + 1] - span[2 * y];
    return wx != wy ? wx > wy : x < y;
  });
  int64_t rows = 0, before = 0;
  for (int b : order) {
    const int64_t start = span[2 * b], stop = span[2 * b + 1];
    const int64_t lq = cu_q[b + 1] - cu_q[b];
    const int64_t step = before * 100 >= (100 - kDecTailPercent) * total ? tail_chunk : chunk;
    before += stop - start;
    dec_seq[2 * b] = static_cast<int32_t>(dec.size());
    int32_t split = 0;
    for (int64_t a = start; a < stop; a += step) {
      Item it{};
      it.w[0] = b;
      it.w[1] = split++;
      it.w[2] = static_cast<int32_t>(a);
      it.w[3] = static_cast<int32_t>(std::min<int64_t>(stop, a + step));
      it.w[4] = static_cast<int32_t>(rows);
      rows += lq * hq;
      dec.push_back(it);
    }
    dec_seq[2 * b + 1] = split;
  }
  return rows;
}

uint32_t fnv1a(const int32_t* a, int64_t n, uint32_t h) {
  const unsigned char* p = reinterpret_cast<const unsigned char*>(a);
  for (int64_t i = 0; i < n * 4; ++i) { h ^= p[i]; h *= 16777619u; }
  return h;
}

}  // namespace

FwdWorkspace fwd_workspace_layout(int64_t dec_rows, int head_dim, int dtype,
                                  int mode) {
  FwdWorkspace w{0, 0, 0, 0};
  // the split-KV partials of the 16-bit (bf16, fp16) decode path; the fp32
  // path has no split mode
  if (dtype == SINK_ATTN_FP32 || mode != kModeDecode) return w;
  w.o_off = 0;
  w.m_off = align_up(dec_rows * head_dim * 4, 256);
  w.l_off = w.m_off + align_up(dec_rows * 4, 256);
  w.bytes = w.l_off + align_up(dec_rows * 4, 256);
  return w;
}

BwdWorkspace bwd_workspace_layout(int64_t total_q, int hq, int head_dim,
                                  int dtype, int64_t pre_blocks) {
  BwdWorkspace w;
  w.dval_off = 0;
  w.part_off = align_up(total_q * hq * 4, 256);
  w.bytes = w.part_off + align_up(pre_blocks * hq * 4, 256);
  (void)head_dim;
  (void)dtype;
  return w;
}

Geometry make_geometry(const sink_attn_problem& p, const int32_t* used_q,
                       const int32_t* used_k) {
  Geometry g{};
  const int64_t hq = p.num_heads_q, hk = p.num_heads_k, d = p.head_dim;
  g.used_q = used_q;
  g.used_k = used_k;
  // Row i of head h of the sequence starting at row r: r*x_seq + i*x_row +
  // h*x_head. TND and BSND ([.., S, N, D]) interleave the heads in a row;
  // BNSD ([B, N, S, D]) keeps each head's S rows together.
  auto set = [&](int layout, int64_t n, int64_t seq, int64_t& xs, int64_t& xr, int64_t& xh) {
    xs = n * d;
    if (layout == SINK_ATTN_BNSD) { xr = d; xh = seq * d; }
    else { xr = n * d; xh = d; }
  };
  set(p.layout_q, hq, p.seq_q, g.q_seq, g.q_row, g.q_head);
  set(p.layout_out, hq, p.seq_q, g.o_seq, g.o_row, g.o_head);
  set(p.layout_q, hk, p.seq_k, g.k_seq, g.k_row, g.k_head);
  if (p.layout_q == SINK_ATTN_TND) {
    // lse [Hq, Tq]
    g.l_seq = 1;
    g.l_row = 1;
    g.l_head = p.total_q;
  } else {
    // lse [B, Hq, S]: sequence b starts at row b*S, b*Hq*S elements in
    g.seq_q = p.seq_q;
    g.seq_k = p.seq_k;
    g.l_seq = hq;
    g.l_row = 1;
    g.l_head = p.seq_q;
  }
  return g;
}

sink_attn_status validate_problem(const sink_attn_problem* p) {
  if (!p) return SINK_ATTN_E_INVALID;
  if (p->batch <= 0 || p->batch >= 65536) return SINK_ATTN_E_INVALID;
  if (p->total_q <= 0 || p->total_k <= 0) return SINK_ATTN_E_INVALID;
  if (p->num_heads_q <= 0 || p->num_heads_k <= 0) return SINK_ATTN_E_INVALID;
  if (p->num_heads_q % p->num_heads_k != 0) return SINK_ATTN_E_INVALID;
  if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return SINK_ATTN_E_INVALID;
  if (p->causal != 0 && p->causal != 1) return SINK_ATTN_E_INVALID;
  if (p->win_left < -1 || p->win_right < -1) return SINK_ATTN_E_INVALID;
  if (p->causal && p->win_right > 0) return SINK_ATTN_E_INVALID;
  if (p->dtype != SINK_ATTN_FP32 && p->dtype != SINK_ATTN_BF16 && p->dtype != SINK_ATTN_FP16)
    return SINK_ATTN_E_UNSUPPORTED;
  // D = 256 runs on the 16-bit MFMA kernels only
  if (p->head_dim != 64 && p->head_dim != 128 &&
      !(p->head_dim == 256 && p->dtype != SINK_ATTN_FP32))
    return SINK_ATTN_E_UNSUPPORTED;
  // layouts: out follows q, except BNSD q with BSND out
  if (p->layout_q != SINK_ATTN_TND && p->layout_q != SINK_ATTN_BSND &&
      p->layout_q != SINK_ATTN_BNSD)
    return SINK_ATTN_E_INVALID;
  if (p->layout_out != p->layout_q &&
      !(p->layout_q == SINK_ATTN_BNSD && p->layout_out == SINK_ATTN_BSND))
    return SINK_ATTN_E_INVALID;
  if (p->layout_q == SINK_ATTN_TND) {
    if (p->seq_q != 0 || p->seq_k != 0) return SINK_ATTN_E_INVALID;
  } else {
    if (p->seq_q <= 0 || p->seq_k <= 0) return SINK_ATTN_E_INVALID;
    if (static_cast<int64_t>(p->batch) * p->seq_q != p->total_q ||
        static_cast<int64_t>(p->batch) * p->seq_k != p->total_k)
      return SINK_ATTN_E_INVALID;
  }
  // element offsets of the largest tensors must fit the kernels' 32-bit
  // row arithmetic
  int64_t rows_q = static_cast<int64_t>(p->total_q) * p->num_heads_q;
  int64_t rows_k = static_cast<int64_t>(p->total_k) * p->num_heads_k;
  if (rows_q * p->head_dim >= (int64_t(1) << 31) * 8 ||
      rows_k * p->head_dim >= (int64_t(1) << 31) * 8)
    return SINK_ATTN_E_UNSUPPORTED;
  return SINK_ATTN_OK;
}

sink_attn_status validate_cu_seqlens(const sink_attn_problem& p,
                                     const int32_t* cu_q, const int32_t* cu_k) {
  if (!cu_q || !cu_k) return SINK_ATTN_E_INVALID;
  if (cu_q[0] != 0 || cu_k[0] != 0) return SINK_ATTN_E_INVALID;
  int32_t mq = 0, mk = 0;
  for (int b = 0; b < p.batch; ++b) {
    int32_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
    if (lq < 0 || lk < 0) return SINK_ATTN_E_INVALID;
    mq = std::max(mq, lq);
    mk = std::max(mk, lk);
  }
  if (cu_q[p.batch] != p.total_q || cu_k[p.batch] != p.total_k)
    return SINK_ATTN_E_INVALID;
  if (mq != p.max_seqlen_q || mk != p.max_seqlen_k) return SINK_ATTN_E_INVALID;
  return SINK_ATTN_OK;
}

sink_attn_status validate_seqused(const sink_attn_problem& p, const int32_t* used_q,
                                  const int32_t* used_k, int32_t* cu_q_out,
                                  int32_t* cu_k_out) {
  if (!cu_q_out || !cu_k_out) return SINK_ATTN_E_INVALID;
  cu_q_out[0] = cu_k_out[0] = 0;
  int32_t mq = 0, mk = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int32_t lq = used_q ? used_q[b] : p.seq_q;
    const int32_t lk = used_k ? used_k[b] : p.seq_k;
    if (lq < 0 || lq > p.seq_q || lk < 0 || lk > p.seq_k) return SINK_ATTN_E_INVALID;
    mq = std::max(mq, lq);
    mk = std::max(mk, lk);
    // at most batch * seq rows in all, which the problem check keeps in int32
    cu_q_out[b + 1] = cu_q_out[b] + lq;
    cu_k_out[b + 1] = cu_k_out[b] + lk;
  }
  if (mq != p.max_seqlen_q || mk != p.max_seqlen_k) return SINK_ATTN_E_INVALID;
  return SINK_ATTN_OK;
}

sink_attn_status validate_paged(const sink_attn_problem& p,
                                const sink_attn_paged_kv* kv,
                                const int32_t* seqused_kv,
                                const int32_t* block_table, int32_t* cu_k_out) {
  if (!kv || !seqused_kv || !block_table || !cu_k_out) return SINK_ATTN_E_INVALID;
  const int64_t bs = kv->block_size;
  if (bs < 16 || bs > 1024 || bs % 16 != 0) return SINK_ATTN_E_INVALID;
  if (kv->max_blocks_per_seq <= 0 || kv->num_blocks <= 0) return SINK_ATTN_E_INVALID;
  if (kv->layout != SINK_ATTN_PA_BBND && kv->layout != SINK_ATTN_PA_BNBD) return SINK_ATTN_E_INVALID;
  int64_t acc = 0;
  cu_k_out[0] = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int64_t used = seqused_kv[b];
    if (used < 0 || used > bs * kv->max_blocks_per_seq) return SINK_ATTN_E_INVALID;
    const int32_t* row = block_table + static_cast<int64_t>(b) * kv->max_blocks_per_seq;
    for (int64_t pg = 0; pg < (used + bs - 1) / bs; ++pg)
      if (row[pg] < 0 || row[pg] >= kv->num_blocks) return SINK_ATTN_E_INVALID;
    acc += used;
    if (acc > std::numeric_limits<int32_t>::max()) return SINK_ATTN_E_INVALID;
    cu_k_out[b + 1] = static_cast<int32_t>(acc);
  }
  return SINK_ATTN_OK;
}

sink_attn_status build_metadata(const sink_attn_problem& p, const int32_t* cu_q,
                                const int32_t* cu_k, const PagedInfo* paged,
                                int used_mask, int32_t* out, int64_t capacity,
                                int64_t* words, int64_t* fwd_ws, int64_t* bwd_ws) {
  const int B = p.batch;
  const int G = p.num_heads_q / p.num_heads_k;
  const int32_t mode =
      (static_cast<int64_t>(p.max_seqlen_q) * G <= kDecMaxRows) ? kModeDecode
                                                                : kModePrefill;
  // Only items some call can read are built. A paged table serves the
  // forward alone: no backward items, and in decode mode (the forward runs
  // the split-KV items) no per-query-tile items either. Other tables keep
  // both, as the backward's dQ pass walks the per-query-tile items. Split-KV
  // items exist in decode mode only (a prefill table would otherwise carry
  // them for nothing, and their partial-row count, query rows x q-heads x
  // key chunks, would cap a single prefill sequence near 370k tokens at 32
  // heads).
  const bool want_bwd = paged == nullptr;
  const bool want_fwd = want_bwd || mode == kModePrefill;
  const bool want_dec = mode == kModeDecode;
  // One forward item per query tile and one backward item per key tile; a
  // call that only asks for the sizes counts them without building them.
  const bool fill = out != nullptr;
  int64_t n_fwd = 0, n_bwd = 0;
  for (int b = 0; b < B; ++b) {
    n_fwd += want_fwd ? (cu_q[b + 1] - cu_q[b] + kFwdBM - 1) / kFwdBM : 0;
    n_bwd += want_bwd ? (cu_k[b + 1] - cu_k[b] + kBwdBN - 1) / kBwdBN : 0;
  }
  std::vector<Item> fwd, bwd, dec;
  if (fill) {
    fwd.reserve(static_cast<size_t>(n_fwd));
    bwd.reserve(static_cast<size_t>(n_bwd));
  }
  std::vector<int32_t> dec_seq(2 * static_cast<size_t>(B), 0);
  std::vector<int64_t> dec_span(2 * static_cast<size_t>(B), 0);   // [start, stop) per sequence
  int64_t dec_rows = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
    const RowBounds rb = row_bounds(p, lq, lk);
    // forward items: one per query tile
    const int64_t nqt = want_fwd && fill ? (lq + kFwdBM - 1) / kFwdBM : 0;
    for (int64_t qt = 0; qt < nqt; ++qt) {
      const int64_t r0 = qt * kFwdBM, r1 = std::min(lq, r0 + kFwdBM);
      Item it{};
      it.w[0] = b;
      it.w[1] = static_cast<int32_t>(qt);
      key_tile_spans(rb, r0, r1, lk, kFwdBM, kFwdBN, it.w + 2);
      fwd.push_back(it);
    }
    // backward items: one per key tile
    const int64_t bbm = bwd_tile_rows(p.head_dim);
    const int64_t bnk = want_bwd && fill ? (lk + kBwdBN - 1) / kBwdBN : 0;
    for (int64_t kt = 0; kt < bnk; ++kt) {
      const int64_t c0 = kt * kBwdBN, c1 = std::min(lk, c0 + kBwdBN);
      Item it{};
      it.w[0] = b;
      it.w[1] = static_cast<int32_t>(kt);
      query_tile_spans(rb, c0, c1, lq, bbm, kBwdBN, it.w + 2);
      bwd.push_back(it);
    }
    // split-KV span: the keys kept by any row (one interval, the rows'
    // intervals being contiguous), rounded out to kDecBN tiles
    if (want_dec && lq > 0 && lk > 0) {
      const int64_t jlo = std::max<int64_t>(0, rb.lo(0));
      const int64_t jhi = std::min<int64_t>(lk - 1, rb.hi(lq - 1)) + 1;
      if (jhi > jlo) {
        dec_span[2 * b] = (jlo / kDecBN) * kDecBN;
        dec_span[2 * b + 1] = std::min<int64_t>(lk, (jhi + kDecBN - 1) / kDecBN * kDecBN);
      }
    }
  }
  sort_items(fwd, B);
  sort_items(bwd, B);
  const int32_t dec_chunk = decode_chunk(dec_span, B, p.num_heads_k);
  const int32_t dec_tail = decode_tail_chunk(dec_span, B, p.num_heads_k, dec_chunk);
  dec_rows = decode_items(dec_span, dec_chunk, dec_tail, B, cu_q, p.num_heads_q, dec, dec_seq);

  const int64_t pre_blocks = (p.total_q + kPreRows - 1) / kPreRows;
  const FwdWorkspace fw = fwd_workspace_layout(dec_rows, p.head_dim, p.dtype, mode);
  const BwdWorkspace bw = bwd_workspace_layout(p.total_q, p.num_heads_q,
                                               p.head_dim, p.dtype, pre_blocks);
  const int64_t dec_off = kHeaderWords;
  const int64_t seq_off = dec_off + static_cast<int64_t>(dec.size()) * kItemWords;
  const int64_t fwd_off = seq_off + 2 * static_cast<int64_t>(B);
  const int64_t bwd_off = fwd_off + n_fwd * kItemWords;
  const int64_t total = bwd_off + n_bwd * kItemWords;
  const int64_t fwd_words = mode == kModeDecode ? fwd_off : bwd_off;
  if (total >= std::numeric_limits<int32_t>::max() ||
      dec_rows >= std::numeric_limits<int32_t>::max())
    return SINK_ATTN_E_UNSUPPORTED;
  if (words) *words = total;
  if (fwd_ws) *fwd_ws = fw.bytes;
  if (bwd_ws) *bwd_ws = bw.bytes;
  if (!out) return SINK_ATTN_OK;
  if (capacity < total) return SINK_ATTN_E_BUFFER_TOO_SMALL;

  std::memset(out, 0, sizeof(int32_t) * kHeaderWords);
  int32_t* h = out;
  h[kMagic] = kMagicValue;
  h[kVersion] = SINK_ATTN_ABI_VERSION;
  h[kBatch] = p.batch;
  h[kHq] = p.num_heads_q;
  h[kHk] = p.num_heads_k;
  h[kHeadDim] = p.head_dim;
  h[kTq] = p.total_q;
  h[kTk] = p.total_k;
  h[kMaxQ] = p.max_seqlen_q;
  h[kMaxK] = p.max_seqlen_k;
  h[kCausal] = p.causal;
  h[kWinL] = p.win_left;
  h[kWinR] = p.win_right;
  h[kDtype] = p.dtype;
  h[kMode] = mode;
  h[kWordFwdBM] = kFwdBM;
  h[kWordFwdBN] = kFwdBN;
  h[kWordBwdBM] = bwd_tile_rows(p.head_dim);
  h[kWordBwdBN] = kBwdBN;
  h[kWordDecBN] = kDecBN;
  h[kWordDecChunk] = dec_chunk;
  h[kWordDecTail] = dec_tail;
  h[kWordDecTailPct] = kDecTailPercent;
  h[kNFwd] = static_cast<int32_t>(n_fwd);
  h[kFwdOff] = static_cast<int32_t>(fwd_off);
  h[kNBwd] = static_cast<int32_t>(n_bwd);
  h[kBwdOff] = static_cast<int32_t>(bwd_off);
  h[kNDec] = static_cast<int32_t>(dec.size());
  h[kDecOff] = static_cast<int32_t>(dec_off);
  h[kDecSeqOff] = static_cast<int32_t>(seq_off);
  h[kDecRows] = static_cast<int32_t>(dec_rows);
  h[kFwdWsLo] = static_cast<int32_t>(fw.bytes & 0xffffffff);
  h[kFwdWsHi] = static_cast<int32_t>(fw.bytes >> 32);
  h[kBwdWsLo] = static_cast<int32_t>(bw.bytes & 0xffffffff);
  h[kBwdWsHi] = static_cast<int32_t>(bw.bytes >> 32);
  h[kCuHash] = static_cast<int32_t>(
      fnv1a(cu_k, B + 1, fnv1a(cu_q, B + 1, 2166136261u)));
  h[kMetaWords] = static_cast<int32_t>(total);
  h[kFwdWords] = static_cast<int32_t>(fwd_words);
  h[kBwdPreBlocks] = static_cast<int32_t>(pre_blocks);
  h[kLayoutQ] = p.layout_q;
  h[kLayoutOut] = p.layout_out;
  h[kSeqQ] = p.seq_q;
  h[kSeqK] = p.seq_k;
  h[kUsedMask] = used_mask;
  if (paged) {
    const int64_t bs = paged->kv.block_size;
    uint32_t hash = 2166136261u;
    for (int b = 0; b < B; ++b) {
      const int64_t used = cu_k[b + 1] - cu_k[b];
      hash = fnv1a(paged->block_table + static_cast<int64_t>(b) * paged->kv.max_blocks_per_seq,
                   (used + bs - 1) / bs, hash);
    }
    h[kPaged] = 1;
    h[kPageSize] = paged->kv.block_size;
    h[kPageMaxBlocks] = paged->kv.max_blocks_per_seq;
    h[kPageNumBlocks] = paged->kv.num_blocks;
    h[kPageLayout] = paged->kv.layout;
    h[kPageHash] = static_cast<int32_t>(hash);
  }
  // per-sequence rows and lengths into words 8-11 of every item
  auto lengths = [&](std::vector<Item>& v) {
    for (Item& it : v) {
      const int b = it.w[0];
      it.w[8] = p.seq_q ? b * p.seq_q : cu_q[b];
      it.w[9] = cu_q[b + 1] - cu_q[b];
      it.w[10] = paged ? 0 : (p.seq_k ? b * p.seq_k : cu_k[b]);
      it.w[11] = cu_k[b + 1] - cu_k[b];
    }
  };
  lengths(dec);
  lengths(fwd);
  lengths(bwd);
  int32_t* w = out + dec_off;
  for (const Item& it : dec) { std::memcpy(w, it.w, sizeof(it.w)); w += kItemWords; }
  std::memcpy(w, dec_seq.data(), sizeof(int32_t) * dec_seq.size());
  w += dec_seq.size();
  for (const Item& it : fwd) { std::memcpy(w, it.w, sizeof(it.w)); w += kItemWords; }
  for (const Item& it : bwd) { std::memcpy(w, it.w, sizeof(it.w)); w += kItemWords; }
  return SINK_ATTN_OK;
}

sink_attn_status check_header(const sink_attn_problem& p, const int32_t* h,
                              const sink_attn_paged_kv* kv) {
  if (!h) return SINK_ATTN_E_INVALID;
  if (h[kMagic] != kMagicValue || h[kVersion] != SINK_ATTN_ABI_VERSION)
    return SINK_ATTN_E_META_MISMATCH;
  if (h[kBatch] != p.batch || h[kHq] != p.num_heads_q ||
      h[kHk] != p.num_heads_k || h[kHeadDim] != p.head_dim ||
      h[kTq] != p.total_q || h[kTk] != p.total_k ||
      h[kMaxQ] != p.max_seqlen_q || h[kMaxK] != p.max_seqlen_k ||
      h[kCausal] != p.causal || h[kWinL] != p.win_left ||
      h[kWinR] != p.win_right || h[kDtype] != p.dtype ||
      h[kLayoutQ] != p.layout_q || h[kLayoutOut] != p.layout_out ||
      h[kSeqQ] != p.seq_q || h[kSeqK] != p.seq_k)
    return SINK_ATTN_E_META_MISMATCH;
  if (h[kWordFwdBM] != kFwdBM || h[kWordFwdBN] != kFwdBN || h[kWordBwdBM] != bwd_tile_rows(p.head_dim) ||
      h[kWordBwdBN] != kBwdBN || h[kWordDecBN] != kDecBN || h[kWordDecChunk] < kDecMinChunk ||
      h[kWordDecChunk] > kDecChunk || h[kWordDecTail] < kDecMinChunk ||
      h[kWordDecTail] > h[kWordDecChunk] || h[kWordDecTailPct] != kDecTailPercent)
    return SINK_ATTN_E_META_MISMATCH;
  if (h[kFwdWords] < kHeaderWords || h[kFwdWords] > h[kMetaWords]) return SINK_ATTN_E_META_MISMATCH;
  if (h[kPaged] != (kv ? 1 : 0)) return SINK_ATTN_E_META_MISMATCH;
  if (kv && (h[kPageSize] != kv->block_size || h[kPageMaxBlocks] != kv->max_blocks_per_seq ||
             h[kPageNumBlocks] != kv->num_blocks || h[kPageLayout] != kv->layout))
    return SINK_ATTN_E_META_MISMATCH;
  return SINK_ATTN_OK;
}

}  // namespace sinkattn
