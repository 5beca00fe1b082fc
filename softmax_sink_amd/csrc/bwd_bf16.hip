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
// Main kernel: one work item = 128 keys of one (sequence, kv-head); wave w
// owns keys 32w..32w+31 and keeps its K and V fragments in registers and
// its dK^T, dV^T accumulators in fp32. It walks the live 64-row query tiles
// of every q-head of the GQA group:
//   S  = Q K^T,  dP = dO V^T        (M = query, N = key; Q, dO from LDS)
//   P  = 2^(S scale log2e - lse log2e), dS = scale P (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS (dO^T, Q^T by transposed LDS reads)
//   dQ += dS K over the item's 128 keys (dS^T staged in LDS), added to an
//   fp32 accumulator with atomics; a final pass converts it to bf16.
#include "bwd_common.h"

namespace sinkattn {
namespace {

using namespace dev;

template <int D>
struct BwdSmem {
  static constexpr int kK = kBwdBN * D * 2;       // K tile [128][D]
  static constexpr int kQ = kBwdBM * D * 2;       // Q tile [64][D]
  static constexpr int kDO = kBwdBM * D * 2;      // dO tile
  static constexpr int kDS = kBwdBN * kBwdBM * 2; // dS^T tile [128 keys][64 q]
  static constexpr int off_k = 0;
  static constexpr int off_q = off_k + kK;
  static constexpr int off_do = off_q + kQ;
  static constexpr int off_ds = off_do + kDO;
  static constexpr int off_lse = off_ds + kDS;    // [64] fp32, log2 domain
  static constexpr int off_dv = off_lse + 256;    // [64] fp32
  static constexpr int bytes = off_dv + 256;
};

// Registers holding the next (q-head, query tile) step's Q, dO, lse, D.
template <int D>
struct QTileLoader {
  static constexpr int kPer = kBwdBM * D / 8 / 256;   // 16-byte chunks per thread
  u32x4 q[kPer], d[kPer];
  float lse2, dval;
  __device__ __forceinline__ void load(const BwdArgs& a, int h, int q0, int lq, int qt) {
    const int64_t stride = (int64_t)a.hq * D;
    const bf16* qp = static_cast<const bf16*>(a.q) + (int64_t)q0 * stride + h * D;
    const bf16* dp = static_cast<const bf16*>(a.dout) + (int64_t)q0 * stride + h * D;
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int u = threadIdx.x + 256 * s;
      const int row = qt * kBwdBM + u / (D / 8), c = u % (D / 8);
      if (row < lq) {
        q[s] = ld16(qp + (int64_t)row * stride + c * 8);
        d[s] = ld16(dp + (int64_t)row * stride + c * 8);
      } else {
        q[s] = u32x4{0u, 0u, 0u, 0u};
        d[s] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (threadIdx.x < kBwdBM) {
      const int row = qt * kBwdBM + threadIdx.x;
      if (row < lq) {
        const float l = a.lse[(int64_t)h * a.total_q + q0 + row];
        // a row with lse = -inf keeps no key: make every P of it 0
        lse2 = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
        dval = a.dval[(int64_t)h * a.total_q + q0 + row];
      } else {
        lse2 = __builtin_huge_valf();
        dval = 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(char* smem) const {
    using S = BwdSmem<D>;
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int u = threadIdx.x + 256 * s;
      lds_store_chunk<D>(smem + S::off_q, u / (D / 8), u % (D / 8), q[s]);
      lds_store_chunk<D>(smem + S::off_do, u / (D / 8), u % (D / 8), d[s]);
    }
    if (threadIdx.x < kBwdBM) {
      reinterpret_cast<float*>(smem + S::off_lse)[threadIdx.x] = lse2;
      reinterpret_cast<float*>(smem + S::off_dv)[threadIdx.x] = dval;
    }
  }
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdArgs a) {
  using S = BwdSmem<D>;
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
  const int hl = lane >> 5, c = lane & 31;
  const int j = kt * kBwdBN + 32 * w + c;        // this lane's key

  const int64_t kstride = (int64_t)a.hk * D;
  const bf16* kp = static_cast<const bf16*>(a.k) + (int64_t)k0 * kstride + hk * D;
  const bf16* vp = static_cast<const bf16*>(a.v) + (int64_t)k0 * kstride + hk * D;

  // K, V fragments as B operands (lane (hl, c) holds row j, columns 16t+8hl..)
  bf16x8 kf[NT], vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (j < lk) {
      kf[t] = __builtin_bit_cast(bf16x8, ld16(kp + (int64_t)j * kstride + 16 * t + 8 * hl));
      vf[t] = __builtin_bit_cast(bf16x8, ld16(vp + (int64_t)j * kstride + 16 * t + 8 * hl));
    } else {
      kf[t] = bf16x8{};
      vf[t] = bf16x8{};
    }
  }
  // K tile in LDS for the dQ product (rows = keys)
  {
    constexpr int kPer = kBwdBN * D / 8 / 256;
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int u = threadIdx.x + 256 * s;
      const int row = u / (D / 8), cc = u % (D / 8);
      const int jj = kt * kBwdBN + row;
      u32x4 v = jj < lk ? ld16(kp + (int64_t)jj * kstride + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      lds_store_chunk<D>(smem + S::off_k, row, cc, v);
    }
  }

  int ilo, ihi;
  key_row_range(j, lq, lk, a.causal, a.win_left, a.win_right, ilo, ihi);

  f32x16 dka[NB], dva[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) { dka[n] = f32x16{}; dva[n] = f32x16{}; }

  const int nq = qt_hi - qt_lo;
  const int steps = nq * G;
  const float c2 = a.scale * kLog2e;
  const float* lse_l = reinterpret_cast<const float*>(smem + S::off_lse);
  const float* dv_l = reinterpret_cast<const float*>(smem + S::off_dv);
  const char* q_l = smem + S::off_q;
  const char* do_l = smem + S::off_do;
  char* ds_l = smem + S::off_ds;
  const int qbw = w >> 1, dh = w & 1;            // this wave's dQ block

  QTileLoader<D> ld;
  if (steps > 0) {
    ld.load(a, hk * G, q0, lq, qt_lo);
    ld.store(smem);
  }
  __syncthreads();

  for (int st = 0; st < steps; ++st) {
    const int g = st / nq, qt = qt_lo + st % nq;
    const int h = hk * G + g;
    const bool more = st + 1 < steps;
    if (more) {
      const int g1 = (st + 1) / nq, qt1 = qt_lo + (st + 1) % nq;
      ld.load(a, hk * G + g1, q0, lq, qt1);
    }

    // S = Q K^T and dP = dO V^T for the two 32-row query blocks
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sc[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sc[qb] = mfma32(lds_row_chunk<D>(q_l, 32 * qb + c, 2 * t + hl), kf[t], sc[qb]);
        dp[qb] = mfma32(lds_row_chunk<D>(do_l, 32 * qb + c, 2 * t + hl), vf[t], dp[qb]);
      }
    }
    // P and dS; query row of slot r is 32qb + 8(r/4) + 4hl + r%4
    const bool partial = qt < qf_lo || qt >= qf_hi;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qq = 32 * qb + 8 * g4 + 4 * hl;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_l + qq);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_l + qq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float p = exp2_hw(__builtin_fmaf(sc[qb][r], c2, -l4[e]));
          if (partial) {
            const int i = qt * kBwdBM + qq + e;
            if (i < ilo || i > ihi) p = 0.f;
          }
          sc[qb][r] = p;
          dp[qb][r] = a.scale * p * (dp[qb][r] - d4[e]);
        }
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the 4 16-row query chunks
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) {
      const bf16x8 pf = frag_half(sc[tq >> 1], tq & 1);
      const bf16x8 sf = frag_half(dp[tq >> 1], tq & 1);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        dva[n] = mfma32(lds_col_operand<D>(do_l, 16 * tq, 32 * n), pf, dva[n]);
        dka[n] = mfma32(lds_col_operand<D>(q_l, 16 * tq, 32 * n), sf, dka[n]);
      }
    }
    // dS^T -> LDS: row = key 32w + c, columns = query rows
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qq = 32 * qb + 8 * g4 + 4 * hl;
        *reinterpret_cast<u32x2*>(ds_l + tile_off<kBwdBM>(32 * w + c, qq)) =
            pack4_bits(dp[qb][4 * g4], dp[qb][4 * g4 + 1], dp[qb][4 * g4 + 2],
                       dp[qb][4 * g4 + 3]);
      }
    __syncthreads();
    if (more) ld.store(smem);       // Q/dO of this step are no longer read

    // dQ[32 rows of block qbw][D/2 columns of half dh] = dS K over 128 keys
#pragma unroll
    for (int nb = 0; nb < D / 64; ++nb) {
      const int col = dh * (D / 2) + 32 * nb;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int tk = 0; tk < kBwdBN / 16; ++tk) {
        const bf16x8 af = lds_col_operand<kBwdBM>(ds_l, 16 * tk, 32 * qbw);
        const bf16x8 bfr = lds_col_operand<D>(smem + S::off_k, 16 * tk, col);
        acc = mfma32(af, bfr, acc);
      }
      float* dqp = a.dq_acc + ((int64_t)q0 * a.hq + h) * D + col + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = qt * kBwdBM + 32 * qbw + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (i < lq) unsafeAtomicAdd(dqp + (int64_t)i * a.hq * D, acc[r]);
      }
    }
    __syncthreads();
  }

  // dK, dV rows of this wave's keys
  if (j < lk) {
    bf16* dkp = static_cast<bf16*>(a.dk) + (int64_t)(k0 + j) * kstride + hk * D;
    bf16* dvp = static_cast<bf16*>(a.dv) + (int64_t)(k0 + j) * kstride + hk * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * n + 8 * g4 + 4 * hl;
        *reinterpret_cast<u32x2*>(dkp + d) =
            pack4_bits(dka[n][4 * g4], dka[n][4 * g4 + 1], dka[n][4 * g4 + 2], dka[n][4 * g4 + 3]);
        *reinterpret_cast<u32x2*>(dvp + d) =
            pack4_bits(dva[n][4 * g4], dva[n][4 * g4 + 1], dva[n][4 * g4 + 2], dva[n][4 * g4 + 3]);
      }
  }
}

// dq = bf16(dq_acc), 8 elements per thread.
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* acc, bf16* dq, int64_t n8) {
  for (int64_t u = blockIdx.x * 256 + threadIdx.x; u < n8; u += (int64_t)gridDim.x * 256) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(acc + 8 * u);
    const f32x4 y = *reinterpret_cast<const f32x4*>(acc + 8 * u + 4);
    *reinterpret_cast<bf16x8*>(dq + 8 * u) = pack8(x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s, const TimingHook& th) {
  hipError_t e = launch_bwd_pre<D, bf16>(a, s);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_main_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, BwdSmem<D>::bytes);
  if (e != hipSuccess) return e;
  if (th.start) hipEventRecord(th.start, s);
  if (a.n_items > 0)
    hipLaunchKernelGGL(bwd_main_kernel<D>, dim3(a.n_items * a.hk), dim3(256),
                       BwdSmem<D>::bytes, s, a);
  if (th.stop) hipEventRecord(th.stop, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n8 = (int64_t)a.total_q * a.hq * D / 8;
  const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 8192);
  hipLaunchKernelGGL(dq_convert_kernel, dim3(blocks), dim3(256), 0, s, a.dq_acc,
                     static_cast<bf16*>(a.dq), n8);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dsink_finalize(a, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, hipStream_t s, const TimingHook& t) {
  return head_dim == 128 ? launch_bwd_d<128>(a, s, t) : launch_bwd_d<64>(a, s, t);
}

}  // namespace sinkattn
