// Backward preprocess and the dsink reduction, shared by the bf16 and fp32
// paths.
//
// "slime: learnable_softmax_attention.py", _LearnableSoftmaxFlashAttnVarlen
// .backward, takes the offset gradient as minus the sum over tokens of
// (dO . O_vanilla) times the derivative of the sigmoid post-scale. With the
// sink-inclusive lse that is the same number as -sum_t p_sink,t D_t with
// p_sink = e^(s - lse) and D_t = dO_t . out_t, which is what is reduced here;
// D_t is also the row term of dS = P (dP - D) in the main backward loop.
#pragma once

#include "device_common.h"
#include "sink_attn_internal.h"
#include "tile_common.h"

namespace sinkattn {
namespace {

// Block (token block bt, q-head h): D = rowsum(dO * out) for kPreRows
// tokens and their -p_sink * D summed in a fixed order into part[h][bt].
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  using namespace dev;
  constexpr int TPR = D / 8;          // threads per token row, 8 elements each
  constexpr int RPP = 256 / TPR;      // rows per pass
  __shared__ float contrib[kPreRows];
  const int bt = blockIdx.x, h = blockIdx.y;
  const int t0 = bt * kPreRows;
  const float sink = a.sinks ? a.sinks[h] : kNegInf;
  const int cidx = threadIdx.x % TPR;
  for (int pass = 0; pass < kPreRows / RPP; ++pass) {
    const int rr = pass * RPP + threadIdx.x / TPR;
    const int t = t0 + rr;
    // row t of the tensors is row i of its sequence; in a padded layout
    // the rows past the sequence's length take no part
    int i = 0;
    bool live = t < a.total_q;
    if (a.g.seq_q && live) {
      int b;
      q_row_of(a, t, b, i);
      live = i < q_len(a, b);
    }
    const int64_t row0 = (int64_t)(t - i);
    float dot = 0.f;
    if (live) {
      const int64_t off = row0 * a.g.o_seq + (int64_t)i * a.g.o_row + h * a.g.o_head + cidx * 8;
      const T* dop = static_cast<const T*>(a.dout) + off;
      const T* op = static_cast<const T*>(a.out) + off;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += (float)dop[e] * (float)op[e];
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    if (cidx == 0) {
      float cterm = 0.f;
      if (t < a.total_q) a.dval[(int64_t)h * a.total_q + t] = dot;
      if (live) {
        const float lse = a.lse[row0 * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head];
        const float ps = sink > kNegInf ? exp2_hw((sink - lse) * kLog2e) : 0.f;
        cterm = -ps * dot;
      }
      contrib[rr] = cterm;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int k = 0; k < kPreRows; ++k) s += contrib[k];
    a.part[(int64_t)h * a.pre_blocks + bt] = s;
  }
}

// dsink[h] = sum over token blocks of part[h][.], fixed order.
__global__ __launch_bounds__(64) void dsink_finalize_kernel(BwdArgs a) {
  const int h = blockIdx.x, lane = threadIdx.x;
  float s = 0.f;
  for (int j = lane; j < a.pre_blocks; j += 64) s += a.part[(int64_t)h * a.pre_blocks + j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0 && a.dsink) a.dsink[h] = s;
}

template <int D, typename T>
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3(a.pre_blocks, a.hq), dim3(256), 0, s, a);
  return hipGetLastError();
}

inline hipError_t launch_dsink_finalize(const BwdArgs& a, hipStream_t s) {
  if (!a.dsink) return hipSuccess;
  hipLaunchKernelGGL(dsink_finalize_kernel, dim3(a.hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace sinkattn
