// Backward kernels, bf16 inputs, fp32 accumulation, for gfx950.
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
//    kv-head), walking the live 64-row query tiles of every q-head of the
//    GQA group; per step
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

template <int D>
struct KvSmem {
  static constexpr int kQ = kBwdBM * D * 2;       // Q tile [64][D]
  static constexpr int off_q = 0;
  static constexpr int off_do = off_q + kQ;       // dO tile
  static constexpr int off_lse = off_do + kQ;     // [64] fp32, log2 domain
  static constexpr int off_dv = off_lse + 256;    // [64] fp32
  static constexpr int stage = off_dv + 256;      // one buffer
  static constexpr int off_p = 2 * stage;         // P^T [128 keys][64 q] fp32
  static constexpr int bytes = off_p + kBwdBN * kBwdBM * 4;
};

constexpr int kKvThreads = 512;                   // 8 waves: 4 key slices x 2 roles

// The next (q-head, query tile) step's Q and dO go straight to LDS; its lse
// and D rows (64 floats each) go through registers.
template <int D>
struct QTileLoader {
  TileDma<D, kKvThreads> q, d;
  float lse, dval;
  bool live;
  int64_t stride;
  __device__ __forceinline__ void init(const BwdArgs& a) {
    stride = (int64_t)a.hq * D;
    q.init();
    d.init();
  }
  __device__ __forceinline__ void load(const BwdArgs& a, int h, int q0, int lq, int qt,
                                       char* buf) {
    using S = KvSmem<D>;
    const bf16* qp = static_cast<const bf16*>(a.q) + (int64_t)q0 * stride + h * D;
    const bf16* dp = static_cast<const bf16*>(a.dout) + (int64_t)q0 * stride + h * D;
    q.load(qp, stride, qt * kBwdBM, lq, buf + S::off_q);
    d.load(dp, stride, qt * kBwdBM, lq, buf + S::off_do);
    if (threadIdx.x < kBwdBM) {
      // raw values only (converting here would wait for the load at once);
      // rows past the sequence read its last row and are flagged
      const int row = qt * kBwdBM + threadIdx.x;
      live = row < lq;
      const int64_t at = (int64_t)h * a.total_q + q0 + min(row, lq - 1);
      lse = a.lse[at];
      dval = a.dval[at];
    }
  }
  __device__ __forceinline__ void store(char* buf) const {
    using S = KvSmem<D>;
    if (threadIdx.x < kBwdBM) {
      // log2-domain lse; rows past the sequence, and rows with lse = -inf
      // (no kept key), get +inf so that every P of them is 0
      reinterpret_cast<float*>(buf + S::off_lse)[threadIdx.x] =
          (!live || lse == kNegInf) ? __builtin_huge_valf() : lse * kLog2e;
      reinterpret_cast<float*>(buf + S::off_dv)[threadIdx.x] = live ? dval : 0.f;
    }
  }
};

// dK/dV, key-tile outer. Waves 0-3 (role 0) own keys 32w..32w+31 of the
// item and compute S = Q K^T, P and dV^T += dO^T P; waves 4-7 (role 1) own
// the same key slices and compute dP = dO V^T, dS = scale P (dP - D) with
// the P that role 0 leaves in LDS, and dK^T += Q^T dS. Each wave holds one
// operand fragment and one accumulator set, so two waves share every SIMD,
// and per SIMD the two roles issue the same number of MFMAs.
template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using S = KvSmem<D>;
  constexpr int NT = D / 16;
  constexpr int NB = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int item = blockIdx.x / a.hk;
  const int hk = blockIdx.x % a.hk;
  const int* it = a.items + item * kItemWords;
  const int b = it[0], kt = it[1], qt_lo = it[2], qt_hi = it[3];
  const int qf_lo = it[4], qf_hi = it[5];
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  const int G = a.group;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int role = w >> 2, kw = w & 3;
  const int hl = lane >> 5, c = lane & 31;
  const int j = kt * kBwdBN + 32 * kw + c;       // this lane's key

  const int64_t kstride = (int64_t)a.hk * D;
  // role 0 holds K rows (B operand of S = Q K^T), role 1 V rows (of dP = dO V^T)
  const bf16* fp = static_cast<const bf16*>(role == 0 ? a.k : a.v) + (int64_t)k0 * kstride + hk * D;
  bf16x8 frag[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    frag[t] = j < lk ? __builtin_bit_cast(bf16x8, ld16(fp + (int64_t)j * kstride + 16 * t + 8 * hl))
                     : bf16x8{};

  int ilo, ihi;
  key_row_range(j, lq, lk, a.causal, a.win_left, a.win_right, ilo, ihi);

  f32x16 acc[NB];                                // role 0: dV^T, role 1: dK^T
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x16{};

  const int nq = qt_hi - qt_lo;
  const int steps = nq * G;
  const float c2 = a.scale * kLog2e;
  char* p_l = smem + S::off_p;

  QTileLoader<D> ld;
  ld.init(a);
  if (steps > 0) {
    ld.load(a, hk * G, q0, lq, qt_lo, smem);
    ld.store(smem);
  }
  wait_vmem();
  __syncthreads();

  // (one copy of the loop body with a run-time buffer offset measures faster
  // here than two copies with constant offsets)
  for (int st = 0; st < steps; ++st) {
    const int stage = st & 1;
    const int qt = qt_lo + st % nq;
    const bool more = st + 1 < steps;
    if (more) ld.load(a, hk * G + (st + 1) / nq, q0, lq, qt_lo + (st + 1) % nq,
                      smem + (stage ^ 1) * S::stage);
    const char* buf = smem + stage * S::stage;
    const char* q_l = buf + S::off_q;
    const char* do_l = buf + S::off_do;
    const float* lse_l = reinterpret_cast<const float*>(buf + S::off_lse);
    const float* dv_l = reinterpret_cast<const float*>(buf + S::off_dv);
    const bool partial = qt < qf_lo || qt >= qf_hi;

    // phase 1: role 0 S = Q K^T -> P (to LDS); role 1 dP = dO V^T.
    // Query row of result slot r of block qb is 32qb + 8(r/4) + 4hl + r%4.
    const char* a_l = role == 0 ? q_l : do_l;
    f32x16 x[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      x[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        x[qb] = mfma32(lds_row_chunk<D>(a_l, 32 * qb + c, 2 * t + hl), frag[t], x[qb]);
    }
    if (role == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qq = 32 * qb + 8 * g4 + 4 * hl;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_l + qq);
          f32x4 p4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p = exp2_hw(__builtin_fmaf(x[qb][4 * g4 + e], c2, -l4[e]));
            if (partial) {
              const int i = qt * kBwdBM + qq + e;
              if (i < ilo || i > ihi) p = 0.f;
            }
            x[qb][4 * g4 + e] = p;
            p4[e] = p;
          }
          *reinterpret_cast<f32x4*>(p_l + tile_off<128>(32 * kw + c, 2 * qq)) = p4;
        }
    }
    __syncthreads();

    // phase 2: role 0 dV^T += dO^T P; role 1 dS = scale P (dP - D), dK^T += Q^T dS
    if (role == 1) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qq = 32 * qb + 8 * g4 + 4 * hl;
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_l + qq);
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(p_l + tile_off<128>(32 * kw + c, 2 * qq));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[qb][4 * g4 + e] = p4[e] * (x[qb][4 * g4 + e] - d4[e]);   // dK scaled at the end
        }
    }
    const char* t_l = role == 0 ? do_l : q_l;
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) {
      const bf16x8 f = frag_half(x[tq >> 1], tq & 1);
#pragma unroll
      for (int n = 0; n < NB; ++n)
        acc[n] = mfma32(lds_col_operand<D>(t_l, 16 * tq, 32 * n), f, acc[n]);
    }
    if (more) ld.store(smem + (stage ^ 1) * S::stage);
    wait_vmem();        // the next Q/dO tile has landed in LDS
    __syncthreads();
  }

  // role 0 writes dV, role 1 dK (times the softmax scale), for this wave's keys
  if (j < lk) {
    bf16* dst = static_cast<bf16*>(role == 0 ? a.dv : a.dk) + (int64_t)(k0 + j) * kstride + hk * D;
    const float sc = role == 0 ? 1.f : a.scale;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * n + 8 * g4 + 4 * hl;
        *reinterpret_cast<u32x2*>(dst + d) =
            pack4_bits(acc[n][4 * g4] * sc, acc[n][4 * g4 + 1] * sc, acc[n][4 * g4 + 2] * sc,
                       acc[n][4 * g4 + 3] * sc);
      }
  }
}

// dQ, query-tile outer. Work items and block numbering are the forward's.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
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
  const int q0 = a.cu_q[b], lq = a.cu_q[b + 1] - q0;
  const int k0 = a.cu_k[b], lk = a.cu_k[b + 1] - k0;
  const int hk = h / a.group;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hl = lane >> 5, c = lane & 31;
  const int i = qt * kFwdBM + w * 32 + c;     // this lane's query row

  const int64_t qstride = (int64_t)a.hq * D;
  const int64_t kstride = (int64_t)a.hk * D;
  const bf16* kp = static_cast<const bf16*>(a.k) + (int64_t)k0 * kstride + hk * D;
  const bf16* vp = static_cast<const bf16*>(a.v) + (int64_t)k0 * kstride + hk * D;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[NT], gf[NT];
  const int64_t roff = (int64_t)(q0 + i) * qstride + h * D;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (i < lq) {
      qf[t] = __builtin_bit_cast(bf16x8, ld16(static_cast<const bf16*>(a.q) + roff + 16 * t + 8 * hl));
      gf[t] = __builtin_bit_cast(bf16x8, ld16(static_cast<const bf16*>(a.dout) + roff + 16 * t + 8 * hl));
    } else {
      qf[t] = bf16x8{};
      gf[t] = bf16x8{};
    }
  }
  float lse2 = __builtin_huge_valf(), dval = 0.f;
  if (i < lq) {
    const float l = a.lse[(int64_t)h * a.total_q + q0 + i];
    lse2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
    dval = a.dval[(int64_t)h * a.total_q + q0 + i];
  }
  const float c2 = a.scale * kLog2e;
  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);

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
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s = mfma32(lds_row_chunk<D>(kt_lds, kb * 32 + c, 2 * t + hl), qf[t], s);
        dp = mfma32(lds_row_chunk<D>(vt_lds, kb * 32 + c, 2 * t + hl), gf[t], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2_hw(__builtin_fmaf(s[r], c2, -lse2));
        if (partial) {
          const int jj = kt * BN + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (jj < jlo || jj > jhi) p = 0.f;
        }
        dp[r] = p * (dp[r] - dval);          // scale is applied to dQ at the end
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x8 sf = frag_half(dp, hh);
#pragma unroll
        for (int n = 0; n < NB; ++n)
          o[n] = mfma32(lds_col_operand<D>(kt_lds, 32 * kb + 16 * hh, 32 * n), sf, o[n]);
      }
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

  if (i < lq) {
    bf16* dqp = static_cast<bf16*>(a.dq) + roff;
    const float sc = a.scale;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * n + 8 * g + 4 * hl;
        *reinterpret_cast<u32x2*>(dqp + d) =
            pack4_bits(o[n][4 * g] * sc, o[n][4 * g + 1] * sc, o[n][4 * g + 2] * sc,
                       o[n][4 * g + 3] * sc);
      }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s, const TimingHook& th) {
  hipError_t e = launch_bwd_pre<D, bf16>(a, s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, KvSmem<D>::bytes);
  if (e != hipSuccess) return e;
  if (th.start) hipEventRecord(th.start, s);
  if (a.n_items > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(a.n_items * a.hk), dim3(kKvThreads),
                       KvSmem<D>::bytes, s, a);
  if (th.stop) hipEventRecord(th.stop, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_items_q > 0)
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(a.n_items_q * a.hq), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dsink_finalize(a, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, hipStream_t s, const TimingHook& t) {
  return head_dim == 128 ? launch_bwd_d<128>(a, s, t) : launch_bwd_d<64>(a, s, t);
}

}  // namespace sinkattn
