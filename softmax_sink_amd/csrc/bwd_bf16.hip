// Backward kernels, bf16 or fp16 inputs (T), fp32 accumulation, for gfx950.
//
// Gradient of the sink softmax ("slime: learnable_softmax_attention.py",
// class docstring and backward; the chain rule through softmax([S, s])):
// the sink column carries a zero value vector, so with the sink-inclusive
// lse the probabilities P = e^(S - lse) and the row term D = dO . out give
// dS = P (dP - D), dP = dO V^T, exactly the vanilla form -- the sink only
// shows up through lse, and as its own gradient -sum p_sink D (bwd_common.h).
// Probabilities are recomputed from lse, never stored ("hf-attention-
// normalizers", Important Limitations: recompute in the fused backward).
//
// Two kernels, neither with atomics:
//  * dK/dV (key-tile outer): one work item = 128 keys of one (sequence,
//    kv-head), walking the live query tiles (64 rows; 32 at D = 256) of
//    every q-head of the GQA group; per step
//      S = Q K^T, dP = dO V^T (M = query, N = key; Q, dO from LDS)
//      P = 2^(S scale log2e - lse log2e), dS = scale P (dP - D)
//      dV^T += dO^T P, dK^T += Q^T dS (dO^T, Q^T by transposed LDS reads)
//    split over two wave roles (see bwd_dkdv_kernel).
//  * dQ (query-tile outer, the shape of the forward kernel): one work item =
//    128 query rows of one (sequence, q-head); each lane owns a query row,
//    so lse and D are per-lane scalars; per 64-key tile
//      S^T = K Q^T, dP^T = V dO^T, dS^T as above, dQ^T += K^T dS^T.
//    Recomputing S and dP here costs 4*D more MFMA work per pair than an
//    atomic dQ update inside the first kernel, and replaces 2.4e9 fp32
//    atomics (plus a zeroed fp32 accumulator) on the long causal workloads;
//    it also makes dQ deterministic.
#include <type_traits>

#include "bwd_common.h"
#include "tile_common.h"

namespace sinkattn {
namespace {

using namespace dev;

// LDS of the dK/dV kernel. Step j of a work item is one (q-head, BM-row
// query tile; BM = 64, or 32 at D = 256 so that the five stages fit). Role 1 works one step behind role 0, so three Q tiles are
// live at once (role 0's, role 1's and the one in flight) and two dO tiles;
// lse and D rows travel with their Q and dO stages. P of a step is handed
// from role 0 to role 1 as 16-bit MFMA fragments ("dumps", one per parity):
// 2 query blocks x 2 halves x 4 key blocks of 32 fragments of 64 lanes x 16 B.
template <int D>
struct KvSmem {
  static constexpr int BM = bwd_tile_rows(D);
  static constexpr int kTile = BM * D * 2;              // one [BM][D] 16-bit tile
  static constexpr int off_q = 0;                       // Q of step j: stage j % 3
  static constexpr int off_do = off_q + 3 * kTile;      // dO of step j: stage j % 2
  static constexpr int off_lse = off_do + 2 * kTile;    // 3 x [64] fp32, log2 domain
  static constexpr int off_dval = off_lse + 3 * 256;    // 2 x [64] fp32
  static constexpr int kDump = (BM / 32) * 8 * 64 * 16;  // one step's P fragments
  static constexpr int off_p = off_dval + 2 * 256;      // P of step j: dump j % 2
  static constexpr int bytes = off_p + 2 * kDump;
};

// 32-key MFMA blocks per wave of the dK/dV kernel. With 2 (4 waves, one per
// SIMD, up to 512 registers each) every LDS operand feeds two MFMAs; with 1
// (8 waves, two per SIMD) each wave needs half the registers and the two
// waves of a SIMD fill each other's waits. 1 is the faster by a fifth on the
// training workloads (4.25 -> 3.38 ms and 3.36 -> 2.57 ms for dK/dV, same
// results bit for bit).
constexpr int kKvKB = 1;
constexpr int kKvWavesPerRole = kBwdBN / (32 * kKvKB);
constexpr int kKvThreads = 64 * 2 * kKvWavesPerRole;

// (q-head offset g, query tile t) of consecutive steps: t runs fastest.
struct StepIdx {
  int g = 0, t = 0;
  __device__ __forceinline__ void next(int nq) {
    if (++t == nq) { t = 0; ++g; }
  }
};

// dK/dV, key-tile outer. With W = kKvWavesPerRole waves per role and
// KB = kKvKB key blocks per wave, wave w owns keys 32*KB*(w % W) .. +32*KB-1
// of the item in role w / W:
//   role 0: S = Q K^T, P = 2^(S scale log2e - lse log2e), dV^T += dO^T P
//   role 1: dP = dO V^T, dS = P (dP - D),                  dK^T += Q^T dS
// With KB = 2 (one wave per SIMD) every operand read from LDS feeds two MFMAs
// (one per key block); with KB = 1 (the build's choice) a SIMD runs two
// waves, which hide each other's waits, at one MFMA per LDS read.
// In iteration i, role 0 computes S and P of step i and the dV update of
// step i-1 (whose P it still holds), so the exponentials of step i can issue
// between the dV MFMAs; role 1 computes all of step i-1 with the P that
// role 0 left in LDS. One barrier per iteration; steps + 1 iterations.
template <int D, typename T>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using S = KvSmem<D>;
  constexpr int BM = S::BM;
  constexpr int QB = BM / 32;                    // 32-row query blocks per step
  constexpr int NT = D / 16;
  constexpr int NB = D / 32;
  constexpr int KB = kKvKB;
  constexpr int W = kKvWavesPerRole;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int item = blockIdx.x / a.hk;
  const int hk = blockIdx.x % a.hk;
  const int* itw = a.items + item * kItemWords;
  const int b = itw[0], kt = itw[1], qt_lo = itw[2], qt_hi = itw[3];
  const int qf_lo = itw[4], qf_hi = itw[5];
  const int q0 = itw[8], lq = itw[9], k0 = itw[10], lk = itw[11];
  const int G = a.group;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int role = w / W, kq = w % W;
  const int hl = lane >> 5, c = lane & 31;
  const int jbase = kt * kBwdBN + 32 * KB * kq + c;  // this lane's key in block kb: jbase + 32 kb

  const int64_t kstride = a.g.k_row;
  const int64_t qstride = a.g.q_row;
  const int64_t koff = (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;   // key row 0 of k / v / dk / dv
  // role 0 holds K rows (B operand of S = Q K^T), role 1 V rows (of dP = dO V^T)
  const T* fp = static_cast<const T*>(role == 0 ? a.k : a.v) + koff;
  vec8<T> frag[KB][NT];
  // kept query rows of each key as start and span of one unsigned range
  // test; a key without rows gets a start above every row index
  int ilo[KB];
  uint32_t ispan[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = jbase + 32 * kb;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      frag[kb][t] = j < lk ? __builtin_bit_cast(vec8<T>, ld16(fp + (int64_t)j * kstride + 16 * t + 8 * hl))
                           : vec8<T>{};
    int lo, hi;
    key_row_range(j, lq, lk, a.causal, a.win_left, a.win_right, lo, hi);
    ilo[kb] = hi < lo ? 1 << 30 : lo;
    ispan[kb] = hi < lo ? 0u : (uint32_t)(hi - lo);
  }

  f32x16 acc[NB][KB];                            // role 0: dV^T, role 1: dK^T
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[n][kb] = f32x16{};
  const int nq = qt_hi - qt_lo;
  const int steps = nq * G;
  const float c2 = a.scale * kLog2e;
  const int64_t qoff = (int64_t)q0 * a.g.q_seq + (int64_t)hk * G * a.g.q_head;
  const T* qg = static_cast<const T*>(a.q) + qoff;     // row 0 of q-head hk*G
  const T* dg = static_cast<const T*>(a.dout) + (int64_t)q0 * a.g.o_seq +
                (int64_t)hk * G * a.g.o_head;   // row 0 of dO of q-head hk*G
  // lse of (q-head hk*G + g, row r): lbase + g*l_head + r*l_row; D (the
  // workspace, [Hq, rows]): rbase + g*total_q + r
  const int64_t lbase = (int64_t)q0 * a.g.l_seq + (int64_t)hk * G * a.g.l_head;
  const int64_t rbase = ((int64_t)hk * G) * a.total_q + q0;
  // P fragment (query block qb, key block kb, half h) of this wave's keys
  const int frag0 = kq * KB;                     // first 32-key block of this wave
  auto dump_at = [&](char* dump, int qb, int kb, int h) __attribute__((always_inline)) {
    return dump + ((((qb * 4 + frag0 + kb) * 2 + h) * 64) + lane) * 16;
  };

  TileDma<D, kKvThreads, BM> dma;
  dma.init();
  // lse / D rows of a step: raw values in registers of wave 0 (converting at
  // once would wait for the load), written to LDS at the end of the iteration
  float lse_raw = 0.f, dval_raw = 0.f;
  bool lse_live = false, dval_live = false;

  if (steps > 0) {
    dma.load(qg, qstride, qt_lo * BM, lq, smem + S::off_q);
    if (threadIdx.x < BM) {
      const int row = qt_lo * BM + threadIdx.x;
      const float l = a.lse[lbase + (int64_t)min(row, lq - 1) * a.g.l_row];
      reinterpret_cast<float*>(smem + S::off_lse)[threadIdx.x] =
          (row >= lq || l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
    }
    // dO stage 1 is read by role 0's (empty) dV update in iteration 0
    for (int o = threadIdx.x * 16; o < S::kTile; o += kKvThreads * 16)
      *reinterpret_cast<u32x4*>(smem + S::off_do + S::kTile + o) = u32x4{};
  }
  wait_vmem();
  __syncthreads();

  StepIdx sq, sd;                                // steps it + 1 (Q) and it (dO)
  sq.next(nq);
  // Start of iteration it: prefetch Q of step it + 1 (into Q stage
  // (it + 1) % 3) and dO of step it (into dO stage it % 2), with their lse
  // and D rows.
  auto prefetch = [&](int it, int qs_next, int ds) __attribute__((always_inline)) {
    if (it + 1 < steps) {
      const int qt = qt_lo + sq.t;
      dma.load(qg + sq.g * a.g.q_head, qstride, qt * BM, lq,
               smem + S::off_q + qs_next * S::kTile);
      if (threadIdx.x < BM) {
        const int row = qt * BM + threadIdx.x;
        lse_live = row < lq;
        lse_raw = a.lse[lbase + (int64_t)sq.g * a.g.l_head + (int64_t)min(row, lq - 1) * a.g.l_row];
      }
    }
    if (it < steps) {
      const int qt = qt_lo + sd.t;
      dma.load(dg + sd.g * a.g.o_head, a.g.o_row, qt * BM, lq,
               smem + S::off_do + ds * S::kTile);
      if (threadIdx.x < BM) {
        const int row = qt * BM + threadIdx.x;
        dval_live = row < lq;
        dval_raw = a.dval[rbase + (int64_t)sd.g * a.total_q + min(row, lq - 1)];
      }
    }
  };
  // End of iteration it: lse / D rows of the prefetched steps (log2-domain
  // lse, +inf for rows past the sequence or with no kept key, so that their
  // P is 0), then wait for the tiles and publish everything.
  auto finish = [&](int it, int qs_next, int ds) __attribute__((always_inline)) {
    if (threadIdx.x < BM) {
      if (it + 1 < steps)
        reinterpret_cast<float*>(smem + S::off_lse + qs_next * 256)[threadIdx.x] =
            (!lse_live || lse_raw == kNegInf) ? __builtin_huge_valf() : lse_raw * kLog2e;
      if (it < steps)
        reinterpret_cast<float*>(smem + S::off_dval + ds * 256)[threadIdx.x] = dval_live ? dval_raw : 0.f;
    }
    wait_vmem();
    __syncthreads();
    sq.next(nq);
    sd.next(nq);
  };

  // The two roles run separate loops with the same barrier sequence (one
  // per iteration), so that each is register-allocated on its own.
  if (steps > 0 && role == 0) {
    vec8<T> pf[QB][KB][2];                         // P of the previous step [qb][kb][half]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) pf[qb][kb][0] = pf[qb][kb][1] = vec8<T>{};
    int qs = 0;                                  // it % 3
    for (int it = 0; it <= steps; ++it) {
      const int qs_next = qs == 2 ? 0 : qs + 1;
      const int ds = it & 1;
      prefetch(it, qs_next, ds);
      const char* q_l = smem + S::off_q + qs * S::kTile;
      const float* lse_l = reinterpret_cast<const float*>(smem + S::off_lse + qs * 256);
      const char* dop_l = smem + S::off_do + (ds ^ 1) * S::kTile;
      char* dump = smem + S::off_p + ds * S::kDump;
      const int qt = qt_lo + sd.t;
      const bool partial = it < steps && (qt < qf_lo || qt >= qf_hi);
      // One 32-row query block at a time: S and P of step it, and the half
      // of the dV update of step it - 1 that uses the same P registers (in
      // iteration 0: zero P against a zeroed tile). Query row of slot r of
      // block qb is 32qb + 8(r/4) + 4hl + r%4. After the last step the Q
      // stage holds stale (or never written) data; that P is never read.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 x[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) x[kb] = f32x16{};
        mfma_priority_high();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const vec8<T> qa = lds_row_chunk<D, T, BM>(q_l, 32 * qb + c, 2 * t + hl);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) x[kb] = mfma32(qa, frag[kb][t], x[kb]);
        }
        sched_mfma_pipeline<KB * NT, KB, 1, 3>();
        if (partial) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = qt * BM + 32 * qb + 8 * (r >> 2) + 4 * hl + (r & 3);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              if ((uint32_t)(i - ilo[kb]) > ispan[kb]) x[kb][r] = kNegInf;
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int db = 0; db < NB; ++db) {
            const vec8<T> da = lds_col_operand<D, T, BM>(dop_l, 16 * (2 * qb + h), 32 * db);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              acc[db][kb] = mfma32(da, pf[qb][kb][h], acc[db][kb]);
          }
        mfma_priority_low();
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_l + 32 * qb + 8 * g4 + 4 * hl);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              x[kb][4 * g4 + e] = exp2_hw(__builtin_fmaf(x[kb][4 * g4 + e], c2, -l4[e]));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            pf[qb][kb][h] = frag_half<T>(x[kb], h);
            *reinterpret_cast<vec8<T>*>(dump_at(dump, qb, kb, h)) = pf[qb][kb][h];
          }
      }
      finish(it, qs_next, ds);
      qs = qs_next;
    }
  } else if (steps > 0) {
    int qs = 0;
    for (int it = 0; it <= steps; ++it) {
      const int qs_next = qs == 2 ? 0 : qs + 1;
      const int qs_prev = qs == 0 ? 2 : qs - 1;  // (it - 1) % 3
      const int ds = it & 1;
      prefetch(it, qs_next, ds);
      if (it > 0) {
        // step it - 1, one 32-row query block at a time:
        // dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS
        const char* do_l = smem + S::off_do + (ds ^ 1) * S::kTile;
        const float* dv_l = reinterpret_cast<const float*>(smem + S::off_dval + (ds ^ 1) * 256);
        const char* qq_l = smem + S::off_q + qs_prev * S::kTile;
        char* dump = smem + S::off_p + (ds ^ 1) * S::kDump;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          f32x16 x[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) x[kb] = f32x16{};
          mfma_priority_high();
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const vec8<T> ga = lds_row_chunk<D, T, BM>(do_l, 32 * qb + c, 2 * t + hl);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) x[kb] = mfma32(ga, frag[kb][t], x[kb]);
          }
          sched_mfma_pipeline<KB * NT, KB, 1, 3>();
          mfma_priority_low();
          vec8<T> pp[KB][2];                      // [kb][half]
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              pp[kb][h] = *reinterpret_cast<const vec8<T>*>(dump_at(dump, qb, kb, h));
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_l + 32 * qb + 8 * g4 + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              // dK is scaled at the end
#pragma unroll
              for (int kb = 0; kb < KB; ++kb)
                x[kb][r] = (float)pp[kb][r >> 3][r & 7] * (x[kb][r] - d4[e]);
            }
          }
          mfma_priority_high();
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            vec8<T> sf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sf[kb] = frag_half<T>(x[kb], h);
#pragma unroll
            for (int db = 0; db < NB; ++db) {
              const vec8<T> qa = lds_col_operand<D, T, BM>(qq_l, 16 * (2 * qb + h), 32 * db);
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) acc[db][kb] = mfma32(qa, sf[kb], acc[db][kb]);
            }
          }
          sched_mfma_pipeline<2 * KB * NB, KB, 2, 2>();
          mfma_priority_low();
        }
      }
      finish(it, qs_next, ds);
      qs = qs_next;
    }
  }

  // role 0 writes dV, role 1 dK (times the softmax scale), each its
  // [128 keys x D] tile through LDS so that the stores write whole rows
  // (both roles at once where the staging buffers hold two tiles, else one
  // after the other)
  static_assert(KB == 1 && W == 4 && kBwdBN == 128, "one 128-key tile per role");
  const float sc = role == 0 ? 1.f : a.scale;
  T* dst = static_cast<T*>(role == 0 ? a.dv : a.dk) + koff + (int64_t)kt * kBwdBN * kstride;
  const int tid = threadIdx.x & 255, nrows = lk - kt * kBwdBN;
  constexpr int kOut = TileRows<D>::kBytes;
  wait_vmem();
  __syncthreads();                              // every wave is done with the LDS stages
  if constexpr (2 * kOut <= S::bytes) {
    tile_rows_to_lds<D, T>(&acc[0][0], sc, smem + role * kOut, tid);
    __syncthreads();
    tile_rows_from_lds<D, T>(smem + role * kOut, dst, kstride, nrows, tid);
  } else {
    static_assert(kOut <= S::bytes, "one tile fits the stages");
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      if (role == rr) tile_rows_to_lds<D, T>(&acc[0][0], sc, smem, tid);
      __syncthreads();
      if (role == rr) tile_rows_from_lds<D, T>(smem, dst, kstride, nrows, tid);
      __syncthreads();
    }
  }
}

// dQ, query-tile outer. Work items and block numbering are the forward's.
template <int D, typename T>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int NT = D / 16;
  constexpr int NB = D / 32;
  constexpr int TILE = BN * D * 2;
  // two buffers as two objects, so that the compiler can tell a prefetch
  // into one from reads of the other and does not wait for the prefetch
  __shared__ __attribute__((aligned(16))) char lds0[2 * TILE];
  __shared__ __attribute__((aligned(16))) char lds1[2 * TILE];

  const int item = blockIdx.x / a.hq;
  const int h = head_of_slot(blockIdx.x % a.hq, a.hq);
  const int* it = a.items_q + item * kItemWords;
  const int b = it[0], qt = it[1], kt_lo = it[2], kt_hi = it[3];
  const int kf_lo = it[4], kf_hi = it[5];
  const int q0 = it[8], lq = it[9], k0 = it[10], lk = it[11];
  const int hk = h / a.group;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hl = lane >> 5, c = lane & 31;
  const int i = qt * kFwdBM + w * 32 + c;     // this lane's query row

  const int64_t kstride = a.g.k_row;
  const T* kp = static_cast<const T*>(a.k) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;
  const T* vp = static_cast<const T*>(a.v) + (int64_t)k0 * a.g.k_seq + hk * a.g.k_head;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T
  vec8<T> qf[NT], gf[NT];
  const int64_t roff = (int64_t)q0 * a.g.q_seq + (int64_t)i * a.g.q_row + h * a.g.q_head;
  const int64_t ooff = (int64_t)q0 * a.g.o_seq + (int64_t)i * a.g.o_row + h * a.g.o_head;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (i < lq) {
      qf[t] = __builtin_bit_cast(vec8<T>, ld16(static_cast<const T*>(a.q) + roff + 16 * t + 8 * hl));
      gf[t] = __builtin_bit_cast(vec8<T>, ld16(static_cast<const T*>(a.dout) + ooff + 16 * t + 8 * hl));
    } else {
      qf[t] = vec8<T>{};
      gf[t] = vec8<T>{};
    }
  }
  float lse2 = __builtin_huge_valf(), dval = 0.f;
  if (i < lq) {
    const float l = a.lse[(int64_t)q0 * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head];
    lse2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
    dval = a.dval[(int64_t)h * a.total_q + q0 + i];
  }
  const float c2 = a.scale * kLog2e;
  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);
  // the partial-tile mask as one unsigned range test; a row without keys
  // gets a start above every key index
  const int jlo_m = jhi < jlo ? 1 << 30 : jlo;
  const uint32_t jspan = jhi < jlo ? 0u : (uint32_t)(jhi - jlo);

  f32x16 o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x16{};

  TileDma<D> kl, vl;
  kl.init();
  vl.init();
  if (kt_lo < kt_hi) {
    kl.load(kp, kstride, kt_lo * BN, lk, lds0);
    vl.load(vp, kstride, kt_lo * BN, lk, lds0 + TILE);
  }
  wait_vmem();
  __syncthreads();

  auto tile_step = [&](auto cur_c, int kt) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    const bool more = kt + 1 < kt_hi;
    if (more) {
      kl.load(kp, kstride, (kt + 1) * BN, lk, cur == 0 ? lds1 : lds0);
      vl.load(vp, kstride, (kt + 1) * BN, lk, (cur == 0 ? lds1 : lds0) + TILE);
    }
    const char* kt_lds = cur == 0 ? lds0 : lds1;
    const char* vt_lds = (cur == 0 ? lds0 : lds1) + TILE;
    const bool partial = kt < kf_lo || kt >= kf_hi;
    // one 32-key block at a time: S^T, dP^T, dS^T, then its two dQ chunks
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      mfma_priority_high();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s = mfma32(lds_row_chunk<D, T>(kt_lds, kb * 32 + c, 2 * t + hl), qf[t], s);
        dp = mfma32(lds_row_chunk<D, T>(vt_lds, kb * 32 + c, 2 * t + hl), gf[t], dp);
      }
      sched_mfma_pipeline<2 * NT, 1, 1, 3>();
      mfma_priority_low();
      // mask (partial tiles only) as S = -inf, so that P is 0: one uniform
      // branch around the whole block rather than one per element, which
      // would cut the softmax into 16 basic blocks
      if (partial) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jj = kt * BN + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if ((uint32_t)(jj - jlo_m) > jspan) s[r] = kNegInf;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_hw(__builtin_fmaf(s[r], c2, -lse2));
        dp[r] = p * (dp[r] - dval);          // scale is applied to dQ at the end
      }
      mfma_priority_high();
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const vec8<T> sf = frag_half<T>(dp, hh);
#pragma unroll
        for (int n = 0; n < NB; ++n)
          o[n] = mfma32(lds_col_operand<D, T>(kt_lds, 32 * kb + 16 * hh, 32 * n), sf, o[n]);
      }
      sched_mfma_pipeline<2 * NB, 1, 2, 2>();
      mfma_priority_low();
    }
    wait_vmem();        // the next tile has landed in LDS
    __syncthreads();
  };
  int kt = kt_lo;
  for (; kt + 1 < kt_hi; kt += 2) {
    tile_step(std::integral_constant<int, 0>{}, kt);
    tile_step(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < kt_hi) tile_step(std::integral_constant<int, 0>{}, kt);

  // dQ (times the softmax scale) through LDS, whole rows per store (the
  // tile buffers are idle: the last step waited for its transfers and synced)
  static_assert(kFwdBM == 128 && kFwdBM * D * 2 <= 2 * TILE, "the dQ tile fits one buffer");
  store_tile_rows<D, T>(o, a.scale, lds0,
                        static_cast<T*>(a.dq) + (int64_t)q0 * a.g.q_seq +
                            (int64_t)qt * kFwdBM * a.g.q_row + h * a.g.q_head,
                        a.g.q_row, lq - qt * kFwdBM);
}

template <int D, typename T>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s, const TimingHook& th) {
  hipError_t e = launch_bwd_pre<D, T>(a, s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, T>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, KvSmem<D>::bytes);
  if (e != hipSuccess) return e;
  hipError_t ev = record_event(th.start, s);
  if (a.n_items > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T>), dim3(a.n_items * a.hk), dim3(kKvThreads),
                       KvSmem<D>::bytes, s, a);
  ev = first_error(ev, record_event(th.stop, s));
  e = first_error(hipGetLastError(), ev);
  if (e != hipSuccess) return e;
  if (a.n_items_q > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, T>), dim3(a.n_items_q * a.hq), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dsink_finalize(a, s);
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a, int head_dim, hipStream_t s, const TimingHook& t) {
  switch (head_dim) {
    case 64: return launch_bwd_d<64, T>(a, s, t);
    case 128: return launch_bwd_d<128, T>(a, s, t);
    default: return launch_bwd_d<256, T>(a, s, t);
  }
}

}  // namespace

hipError_t launch_bwd_16(const BwdArgs& a, int head_dim, int dtype, hipStream_t s,
                         const TimingHook& t) {
  return dtype == SINK_ATTN_FP16 ? launch_bwd_t<f16>(a, head_dim, s, t)
                                 : launch_bwd_t<bf16>(a, head_dim, s, t);
}

}  // namespace sinkattn
