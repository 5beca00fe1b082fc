// Forward kernels, bf16 or fp16 inputs (T), fp32 softmax state, for gfx950.
//
// Method: "slime: learnable_softmax_attention.py" (module docstring) defines
// the probabilities as softmax over [scores, sink] with the sink column
// dropped; "CANN ops-transformer: flash_attn" (Formula section) writes the
// same thing in max-stabilised form m = max(sink, max S). The tile loop
// keeps that form online: the running max starts at the sink logit and the
// running denominator at e^(sink - m) = 1, so the sink enters exactly once
// and the tiles only ever add real keys -- the virtual logit / zero-value
// sink of "hf-attention-normalizers" (Important Limitations). The returned
// lse includes the sink; the backward recomputes P = e^(S - lse) from it.
//
// Prefill kernel (one work item = 128 query rows of one (sequence, q-head)):
// 4 waves x 32 rows. Per 64-key tile, K and V are staged HBM -> LDS
// (double buffered, 16-byte coalesced loads, swizzled rows) and each wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}, so that every lane
// owns one query row: the row max needs one exchange with lane ^ 32, the
// rescale factor is a per-lane scalar, and the probabilities are already the
// B operand of O^T += V^T P^T (V^T read with ds_read_b64_tr_b16). Only tiles
// that the schedule marks partial evaluate the mask.
//
// Split-KV kernel (short query groups): one work item = one (sequence,
// kv-head, key chunk); all (query row, q-head of the group) pairs, at most
// 64, share every K/V tile, which is read from HBM exactly once. Each item
// writes unnormalised partial (O, m, l) without the sink; the combine kernel
// merges the chunks by their maxima and adds e^(sink) once.
#include <type_traits>

#include "tile_common.h"

namespace sinkattn {
namespace {

using namespace dev;


// Block-table entries a kernel keeps in LDS: those of one split-KV chunk
// (kDecChunk keys) or of one kPageSpan-key span of the tiled forward, at the
// smallest block size (16).
constexpr int kPageSpan = 2048;
constexpr int kMaxItemPages = 260;
static_assert(kMaxItemPages >= 1 + (kDecChunk + 14) / 16 && kMaxItemPages >= 1 + (kPageSpan + 14) / 16,
              "page list too short");

// PAGED: keys and values come from paged caches through the block table
// (only the tile addresses change). The block-table entries of the current
// kPageSpan-key span of the sequence sit in LDS and are refilled when the
// tile prefetch crosses into the next span.
template <int D, typename T, bool PAGED>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void fwd_prefill_kernel(FwdArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int NT = D / 16;            // K chunks of the QK^T product
  constexpr int NB = D / 32;            // 32-column blocks of O^T
  constexpr int TILE = BN * D * 2;      // bytes per K or V tile
  static_assert(kPageSpan % BN == 0, "tiles do not straddle page spans");
  // two buffers as two objects, so that the compiler can tell a prefetch
  // into one from reads of the other and does not wait for the prefetch
  __shared__ __attribute__((aligned(16))) char lds0[2 * TILE];
  __shared__ __attribute__((aligned(16))) char lds1[2 * TILE];
  __shared__ int pages[PAGED ? kMaxItemPages : 1];

  const int item = blockIdx.x / a.hq;
  const int h = head_of_slot(blockIdx.x % a.hq, a.hq);
  const int* it = a.items + item * kItemWords;
  const int b = it[0], qt = it[1], kt_lo = it[2], kt_hi = it[3];
  const int kf_lo = it[4], kf_hi = it[5];
  const int q0 = it[8], lq = it[9], k0 = it[10], lk = it[11];
  const int hk = h / a.group;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hl = lane >> 5, c = lane & 31;
  const int i = qt * kFwdBM + w * 32 + c;     // this lane's query row

  const int64_t qstride = a.g.q_row;
  const int64_t kstride = a.g.k_row;
  const int64_t qoff = (int64_t)q0 * a.g.q_seq + h * a.g.q_head;   // row 0 of q
  const T* qp = static_cast<const T*>(a.q) + qoff;
  const T* kp = static_cast<const T*>(a.k) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;
  const T* vp = static_cast<const T*>(a.v) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;

  // Q as the B operand of S^T = K Q^T: lane (hl, c) holds Q[i][16t + 8hl .. +7]
  vec8<T> qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (i < lq) qf[t] = __builtin_bit_cast(vec8<T>, ld16(qp + (int64_t)i * qstride + 16 * t + 8 * hl));
    else qf[t] = vec8<T>{};
  }

  const float sink = a.sinks ? a.sinks[h] : kNegInf;
  const float c2 = a.scale * kLog2e;         // scores -> log2 domain
  float m = sink * kLog2e;                   // running max (log2 domain)
  float l = (hl == 0 && sink > kNegInf) ? 1.f : 0.f;   // e^(sink - m), counted once
  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);
  // the partial-tile mask as one unsigned range test; a row without keys
  // gets a start above every key index, so that every j - jlo wraps high
  const int jlo_m = jhi < jlo ? 1 << 30 : jlo;
  const uint32_t jspan = jhi < jlo ? 0u : (uint32_t)(jhi - jlo);

  TileDma<D> kl, vl;
  PagedTileDma<D> pl;
  kl.init();
  vl.init();
  pl.init();
  // paged: block-table entries of the span holding key `key0` into LDS
  // (the caller syncs before: no tile of the previous span is being issued)
  int span0 = -1, off0 = 0;
  auto fill_pages = [&](int key0) __attribute__((always_inline)) {
    span0 = key0 / kPageSpan * kPageSpan;
    const int p0 = span0 / a.page_size;
    off0 = span0 - p0 * a.page_size;
    const int span1 = min(lk, span0 + kPageSpan);
    const int np = (off0 + span1 - span0 + a.page_size - 1) / a.page_size;
    const int* bt = a.block_table + (int64_t)b * a.page_cols + p0;
    for (int t = threadIdx.x; t < np; t += 256) pages[t] = bt[t];
    __syncthreads();
  };
  // K and V rows [row0, row0 + BN) into one LDS buffer
  auto load_kv = [&](int row0, char* dst) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int last = min(lk, span0 + kPageSpan) - 1;
      pl.load_kv(static_cast<const T*>(a.k), static_cast<const T*>(a.v), hk * a.page_head, a.page_row,
                 a.page_stride, pages, off0, span0, row0, last, a.page_size, a.page_magic, dst,
                 dst + TILE);
    } else {
      kl.load(kp, kstride, row0, lk, dst);
      vl.load(vp, kstride, row0, lk, dst + TILE);
    }
  };
  if (kt_lo < kt_hi) {
    if constexpr (PAGED) fill_pages(kt_lo * BN);
    load_kv(kt_lo * BN, lds0);
  }
  wait_vmem();
  __syncthreads();

  // One 64-key tile; CUR (the LDS buffer) is a compile-time constant so that
  // every LDS address is a per-lane base plus an immediate.
  auto tile_step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value;
    const bool more = kt + 1 < kt_hi;
    if (more) {
      if constexpr (PAGED) {
        // every wave issued tile kt (in the previous step) before the
        // barrier that ended it, so the page list may be replaced now
        if ((kt + 1) * BN >= span0 + kPageSpan) fill_pages((kt + 1) * BN);
      }
      load_kv((kt + 1) * BN, CUR == 0 ? lds1 : lds0);
    }
    const char* kt_lds = CUR == 0 ? lds0 : lds1;
    const char* vt_lds = (CUR == 0 ? lds0 : lds1) + TILE;

    // S^T for the two 32-key blocks of the tile
    f32x16 s[2] = {f32x16{}, f32x16{}};
    mfma_priority_high();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma32(lds_row_chunk<D, T>(kt_lds, kb * 32 + c, 2 * t + hl), qf[t], s[kb]);
    }
    sched_mfma_pipeline<2 * NT, 1, 1, 3>();
    mfma_priority_low();

    // mask (partial tiles only): key of slot r is kt*BN + 32kb + 8(r/4) + 4hl + r%4
    if (kt < kf_lo || kt >= kf_hi) {
      const int d0 = kt * BN + 4 * hl - jlo_m;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((uint32_t)(d0 + kb * 32 + 8 * (r >> 2) + (r & 3)) > jspan) s[kb][r] = kNegInf;
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = half_max(mx);
    // The running max follows the exact row max, so the largest P of a row
    // is exactly 1 in 16 bits (few-key rows keep their accuracy); O and l are
    // rescaled only when some lane's max moved.
    const float m_new = fmaxf(m, mx * c2);
    const bool move = m_new > m;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m - m_use);
    m = m_new;
    // P (fp32 row sum, so that lse keeps fp32 accuracy; 16-bit as the B
    // operand of the PV product)
    vec8<T> pf[4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16& st = s[t >> 1];
      const int o8 = 8 * (t & 1);
      float e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        e[u] = exp2_hw(__builtin_fmaf(st[o8 + u], c2, -m_use));
        psum += e[u];
      }
      pf[t] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    if (__any(move)) {
      l *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
    }
    l += psum;

    // O^T += V^T P^T over the 4 16-key chunks of the tile
    mfma_priority_high();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int n = 0; n < NB; ++n)
        o[n] = mfma32(lds_col_operand<D, T>(vt_lds, 16 * t, 32 * n), pf[t], o[n]);
    }
    sched_mfma_pipeline<4 * NB, 1, 2, 2>();
    mfma_priority_low();

    wait_vmem();        // the next tile has landed in LDS
    __syncthreads();
  };
  int kt = kt_lo;
  for (; kt + 1 < kt_hi; kt += 2) {
    tile_step(std::integral_constant<int, 0>{}, kt);
    tile_step(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < kt_hi) tile_step(std::integral_constant<int, 0>{}, kt);

  // epilogue: out = O / l, lse = m + log2(l) (natural log), sink included;
  // O goes through LDS (the tile buffers are idle: the last step waited for
  // its transfers and synced) so that the stores write whole rows
  const float lt = l + half_partner(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (i < lq && hl == 0)
    a.lse[(int64_t)q0 * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head] =
        lt > 0.f ? (m + log2_hw(lt)) * kLn2 : kNegInf;
  static_assert(kFwdBM == 128 && kFwdBM * D * 2 <= 2 * TILE, "the O tile fits one buffer");
  store_tile_rows<D, T>(o, inv, lds0,
                        static_cast<T*>(a.out) + (int64_t)q0 * a.g.o_seq +
                            (int64_t)qt * kFwdBM * a.g.o_row + h * a.g.o_head,
                        a.g.o_row, lq - qt * kFwdBM);
}

// ---------------------------------------------------------------------------
// Split-KV forward for short query groups.
// Wave w: query block qb = w & 1 (rows 32qb..32qb+31 of the group), key half
// kh = w >> 1 (keys 32kh..32kh+31 of each 64-key tile). Group row r = g*Lq+i
// is query row i of q-head hk*G + g. PAGED: keys and values come from paged
// caches through the block table (only the tile addresses change).
// ---------------------------------------------------------------------------

template <int D, typename T, bool PAGED>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void fwd_split_kernel(FwdArgs a) {
  constexpr int BN = kDecBN;
  constexpr int NT = D / 16;
  constexpr int NB = D / 32;
  constexpr int TILE = BN * D * 2;
  // two buffers as two objects (see fwd_prefill_kernel)
  __shared__ __attribute__((aligned(16))) char lds0[2 * TILE];
  __shared__ __attribute__((aligned(16))) char lds1[2 * TILE];
  __shared__ int pages[PAGED ? kMaxItemPages : 1];

  int item, hk;
  chunk_work(blockIdx.x, a.n_items, a.hk, item, hk);
  const int* it = a.items + item * kItemWords;
  const int b = it[0], k_lo = it[2], k_hi = it[3], row_base = it[4];
  const int q0 = it[8], lq = it[9], k0 = it[10], lk = it[11];
  const int G = a.group;
  const int rows = lq * G;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hl = lane >> 5, c = lane & 31;
  const int qb = w & 1, kh = w >> 1;
  const int r = qb * 32 + c;                 // this lane's group row
  const int g = lq > 0 ? r / lq : 0, i = lq > 0 ? r % lq : 0;
  const int h = hk * G + g;

  const int64_t kstride = a.g.k_row;
  const T* kp = static_cast<const T*>(a.k) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;
  const T* vp = static_cast<const T*>(a.v) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;

  vec8<T> qf[NT];
  const bool live_row = r < rows;
  const T* qrow = static_cast<const T*>(a.q) + (int64_t)q0 * a.g.q_seq + (int64_t)i * a.g.q_row +
                  h * a.g.q_head;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qf[t] = live_row ? __builtin_bit_cast(vec8<T>, ld16(qrow + 16 * t + 8 * hl)) : vec8<T>{};

  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);
  if (!live_row) jhi = -1;
  // Keys every live row of this wave keeps (rows past the group do not
  // count: nothing of theirs is written). A tile inside [wlo, whi] needs no
  // mask; at decode shapes that is every tile but the ones at a sequence's
  // end, window or chunk edge.
  int wlo = live_row ? jlo : INT32_MIN;
  int whi = live_row ? min(jhi, k_hi - 1) : INT32_MAX;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    wlo = max(wlo, __shfl_xor(wlo, o));
    whi = min(whi, __shfl_xor(whi, o));
  }

  const float c2 = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;
  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  const int nt = (k_hi - k_lo + BN - 1) / BN;
  TileDma<D> kl;
  PagedTileDma<D> pl;
  kl.init();
  pl.init();
  int off0 = 0;
  if constexpr (PAGED) {
    // block-table entries of the pages holding keys [k_lo, k_hi)
    const int p0 = k_lo / a.page_size;
    off0 = k_lo - p0 * a.page_size;
    const int np = (off0 + k_hi - k_lo + a.page_size - 1) / a.page_size;
    const int* bt = a.block_table + (int64_t)b * a.page_cols + p0;
    for (int t = threadIdx.x; t < np; t += 256) pages[t] = bt[t];
    __syncthreads();
  }
  // K and V rows [row0, row0 + BN) of the item into one LDS buffer
  auto load_kv = [&](int row0, char* dst) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      pl.load_kv(static_cast<const T*>(a.k), static_cast<const T*>(a.v), hk * a.page_head, a.page_row,
                 a.page_stride, pages, off0, k_lo, row0, k_hi - 1, a.page_size, a.page_magic, dst,
                 dst + TILE);
    } else {
      kl.load(kp, kstride, row0, k_hi, dst);
      kl.load(vp, kstride, row0, k_hi, dst + TILE);
    }
  };
  if (nt > 0) load_kv(k_lo, lds0);
  wait_vmem();
  __syncthreads();

  auto tile_step = [&](auto cur_c, int n_t) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    const bool more = n_t + 1 < nt;
    const int base = k_lo + n_t * BN;
    if (more) load_kv(base + BN, cur == 0 ? lds1 : lds0);
    const char* kt_lds = cur == 0 ? lds0 : lds1;
    const char* vt_lds = (cur == 0 ? lds0 : lds1) + TILE;
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      vec8<T> kf = lds_row_chunk<D, T>(kt_lds, kh * 32 + c, 2 * t + hl);
      s = mfma32(kf, qf[t], s);
    }
    const int tlo = base + kh * 32;              // this wave's 32 keys of the tile
    if (tlo < wlo || tlo + 31 > whi) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = tlo + 8 * (rr >> 2) + 4 * hl + (rr & 3);
        if (j < jlo || j > jhi || j >= k_hi) s[rr] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
    mx = half_max(mx);
    const float m_new = fmaxf(m, mx * c2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m - m_use);
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = exp2_hw(__builtin_fmaf(s[rr], c2, -m_use));
      s[rr] = p;
      psum += p;
    }
    l = l * alpha + psum;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const vec8<T> pf = frag_half<T>(s, t);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const vec8<T> vf = lds_col_operand<D, T>(vt_lds, kh * 32 + 16 * t, 32 * n);
        o[n] = mfma32(vf, pf, o[n]);
      }
    }
    wait_vmem();        // the next tile has landed in LDS
    __syncthreads();
  };
  int n_t = 0;
  for (; n_t + 1 < nt; n_t += 2) {
    tile_step(std::integral_constant<int, 0>{}, n_t);
    tile_step(std::integral_constant<int, 1>{}, n_t + 1);
  }
  if (n_t < nt) tile_step(std::integral_constant<int, 0>{}, n_t);

  // merge the two key halves: waves 2,3 hand (m, l, O) to waves 0,1
  l = l + half_partner(l);
  // (both buffers are idle: the last step waited for its loads and synced)
  float* xo = reinterpret_cast<float*>(lds0);        // [2 waves][NB*16][64 lanes]: all of lds0
  float* xm = reinterpret_cast<float*>(lds1);        // [2 waves][64 lanes]
  float* xl = xm + 2 * 64;
  static_assert(2 * NB * 16 * 64 * 4 <= 2 * TILE, "O exchange fits one buffer");
  if (kh == 1) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) xo[(qb * NB * 16 + n * 16 + rr) * 64 + lane] = o[n][rr];
    xm[qb * 64 + lane] = m;
    xl[qb * 64 + lane] = l;
  }
  __syncthreads();
  if (kh == 0 && live_row) {
    const float m1 = xm[qb * 64 + lane], l1 = xl[qb * 64 + lane];
    const float mt = fmaxf(m, m1);
    const float mu = mt == kNegInf ? 0.f : mt;
    const float f0 = exp2_hw(m - mu), f1 = exp2_hw(m1 - mu);
    const int prow = row_base + h * lq + i;
    float* po = a.ws_o + (int64_t)prow * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * n + 8 * gq + 4 * hl;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = o[n][4 * gq + e] * f0 + xo[(qb * NB * 16 + n * 16 + 4 * gq + e) * 64 + lane] * f1;
        *reinterpret_cast<f32x4*>(po + d) = v;
      }
    if (hl == 0) {
      a.ws_m[prow] = mt;
      a.ws_l[prow] = l * f0 + l1 * f1;
    }
  }
}

// One wave per (token, q-head) row: merge the chunk partials of its sequence
// by their maxima, add the sink once, normalise. The wave's lanes work side
// by side so that the row costs a few memory latencies rather than a chain
// of them: a 64-way search finds the sequence of a packed token (one round
// for up to 64 sequences), lane j reads the (m, l) partials of chunk j, and
// the O partials of all chunks are then requested back to back, each
// chunk's row and weight broadcast from its lane. Sums run in a fixed order.
template <int D, typename T>
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.total_q * a.hq) return;
  const int t = row / a.hq, h = row % a.hq;
  int b, i;                                     // sequence and row of token t
  if (a.g.seq_q) {
    b = t / a.g.seq_q;
    i = t - b * a.g.seq_q;
  } else {
    // cu_q[lo] <= t < cu_q[hi] throughout; lane 0 always tests cu_q[lo]
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int step = (hi - lo + 63) / 64;
      const int idx = lo + lane * step;
      const bool below = idx < hi && a.cu_q[idx] <= t;
      const int j = 63 - __builtin_clzll(__ballot(below));
      const int nlo = lo + j * step;
      hi = min(nlo + step, hi);
      lo = nlo;
    }
    b = lo;
    i = t - a.cu_q[b];
  }
  const int q0 = q_start(a, b), lq = q_len(a, b);
  if (i >= lq) return;                          // padding of a padded layout
  const int first = a.dec_seq[2 * b], n = a.dec_seq[2 * b + 1];
  const float sink = a.sinks ? a.sinks[h] : kNegInf;
  // Chunks eight at a time: lane u < 8 reads the row base of chunk g + u,
  // then the (m, l) of that chunk and, across all lanes, the O partials of
  // all eight chunks go out together, so that a row of up to eight chunks
  // costs one dependent load after its row bases. A running maximum merges
  // the groups (O and l rescaled when it grows); sums in a fixed order.
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float lpart = 0.f;
  float mt = sink * kLog2e;                     // running maximum, the sink included
  for (int g = 0; g < n; g += 8) {
    const int cnt = min(8, n - g);
    int prow = 0;
    if (lane < cnt) prow = a.items[(first + g + lane) * kItemWords + 4] + h * lq + i;
    float v[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // a slot past the last chunk re-reads chunk 0 of the group (weight 0)
      const float* po = a.ws_o + (int64_t)__builtin_amdgcn_readlane(prow, u < cnt ? u : 0) * D + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[u][e] = po[e];
    }
    float mc = kNegInf, lc = 0.f;
    if (lane < cnt) {
      mc = a.ws_m[prow];
      lc = a.ws_l[prow];
    }
    float gm = mc;
    for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
    const float m_new = fmaxf(mt, gm);
    const float mu = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(mt - mu);       // 0 while nothing was counted
    const float f = exp2_hw(mc - mu);           // 0 for lanes past the group
    mt = m_new;
    lpart = lpart * alpha + lc * f;
    const int fbits = __float_as_int(f);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float fu = u < cnt ? __int_as_float(__builtin_amdgcn_readlane(fbits, u)) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += v[u][e] * fu;
    }
  }
  const float mu = mt == kNegInf ? 0.f : mt;
  for (int o = 32; o > 0; o >>= 1) lpart += __shfl_xor(lpart, o);
  const float lt = lpart + exp2_hw(sink * kLog2e - mu);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  T* op = static_cast<T*>(a.out) + (int64_t)q0 * a.g.o_seq + (int64_t)i * a.g.o_row +
          h * a.g.o_head + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[e] = (T)(acc[e] * inv);
  if (lane == 0)
    a.lse[(int64_t)q0 * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head] =
        lt > 0.f ? (mt + log2_hw(lt)) * kLn2 : kNegInf;
}

template <int D, typename T>
hipError_t launch_fwd_d(const FwdArgs& a, int mode, hipStream_t s, const TimingHook& th) {
  hipError_t ev = record_event(th.start, s);
  if (mode == kModeDecode) {
    if (a.n_items > 0) {
      if (a.block_table)
        hipLaunchKernelGGL((fwd_split_kernel<D, T, true>), dim3(a.n_items * a.hk), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((fwd_split_kernel<D, T, false>), dim3(a.n_items * a.hk), dim3(256), 0, s, a);
    }
    ev = first_error(ev, record_event(th.stop, s));
    const int rows = a.total_q * a.hq;
    hipLaunchKernelGGL((fwd_combine_kernel<D, T>), dim3((rows + 3) / 4), dim3(256), 0, s, a);
  } else {
    if (a.block_table)
      hipLaunchKernelGGL((fwd_prefill_kernel<D, T, true>), dim3(a.n_items * a.hq), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fwd_prefill_kernel<D, T, false>), dim3(a.n_items * a.hq), dim3(256), 0, s, a);
    ev = first_error(ev, record_event(th.stop, s));
  }
  return first_error(hipGetLastError(), ev);
}

template <typename T>
hipError_t launch_fwd_t(const FwdArgs& a, int head_dim, int mode, hipStream_t s,
                        const TimingHook& t) {
  switch (head_dim) {
    case 64: return launch_fwd_d<64, T>(a, mode, s, t);
    case 128: return launch_fwd_d<128, T>(a, mode, s, t);
    default: return launch_fwd_d<256, T>(a, mode, s, t);
  }
}

}  // namespace

hipError_t launch_fwd_16(const FwdArgs& a, int head_dim, int dtype, int mode, hipStream_t s,
                         const TimingHook& t) {
  return dtype == SINK_ATTN_FP16 ? launch_fwd_t<f16>(a, head_dim, mode, s, t)
                                 : launch_fwd_t<bf16>(a, head_dim, mode, s, t);
}

}  // namespace sinkattn
