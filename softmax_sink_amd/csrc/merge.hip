// Context-parallel merge of sink-free partial results.
//
// "CANN ops-transformer: flash_attn", Note on softmax_lse: the returned lse
// is what ring attention combines partial results with. When the keys of a
// sequence are split into disjoint parts (for instance across the ranks of a
// ring), each part yields out_p, the softmax attention over its keys alone
// without the sink, and lse_p = ln sum e^S over those keys. The attention
// over all keys WITH the sink ("CANN", Formula section; "slime", module
// docstring) follows from these alone, the sink entering exactly once:
//   lse = ln(e^s + sum_p e^{lse_p}),   out = sum_p e^{lse_p - lse} out_p.
// Evaluated max-stabilised in the log2 domain, in fp32.
#include "device_common.h"
#include "sink_attn_internal.h"

namespace sinkattn {
namespace {

using namespace dev;

// Eight consecutive elements as fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const u32x4 v = ld16(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(v[e] << 16);
    x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
__device__ __forceinline__ void load8(const f16* p, float (&x)[8]) {
  const f16x8 v = __builtin_bit_cast(f16x8, ld16(p));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(
      u32x4, pack8<T>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]));
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// D/8 lanes per (token, q-head) row, eight elements per lane, so a wave
// moves whole 16-byte chunks of several rows; parts are read four at a time
// so that several loads per lane are in flight.
template <int D, typename TP, typename TO>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 8;                  // lanes per row
  constexpr int RPB = 256 / LPR;              // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int col = (threadIdx.x % LPR) * 8;
  const int64_t rows = (int64_t)a.total_q * a.hq;
  if (row >= rows) return;
  const int64_t t = row / a.hq;
  const int h = (int)(row % a.hq);
  const float sink2 = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  const float* lp = a.part_lse + (int64_t)h * a.total_q + t;
  const int64_t lstride = (int64_t)a.hq * a.total_q;
  float m = sink2;
  for (int p = 0; p < a.parts; ++p) m = fmaxf(m, lp[p * lstride] * kLog2e);
  const float mu = m == kNegInf ? 0.f : m;
  float lt = exp2_hw(sink2 - mu);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const TP* po = static_cast<const TP*>(a.part_out) + row * D + col;
  const int64_t pstride = rows * D;
  int p = 0;
  for (; p + 4 <= a.parts; p += 4) {
    float x[4][8], w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      load8(po + (p + u) * pstride, x[u]);
      w[u] = exp2_hw(lp[(p + u) * lstride] * kLog2e - mu);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lt += w[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w[u] * x[u][e];
    }
  }
  for (; p < a.parts; ++p) {
    float x[8];
    load8(po + p * pstride, x);
    const float w = exp2_hw(lp[p * lstride] * kLog2e - mu);
    lt += w;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * x[e];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8(static_cast<TO*>(a.out) + row * D + col, acc);
  if (col == 0) a.lse[(int64_t)h * a.total_q + t] = lt > 0.f ? (mu + log2_hw(lt)) * kLn2 : kNegInf;
}

template <int D, typename TP>
hipError_t launch_d(const MergeArgs& a, int out_dtype, hipStream_t s) {
  const int64_t rows = (int64_t)a.total_q * a.hq;
  constexpr int RPB = 256 / (D / 8);
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  if (out_dtype == SINK_ATTN_BF16)
    hipLaunchKernelGGL((merge_kernel<D, TP, bf16>), grid, dim3(256), 0, s, a);
  else if (out_dtype == SINK_ATTN_FP16)
    hipLaunchKernelGGL((merge_kernel<D, TP, f16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, TP, float>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TP>
hipError_t launch_tp(const MergeArgs& a, int head_dim, int out_dtype, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<64, TP>(a, out_dtype, s);
    case 128: return launch_d<128, TP>(a, out_dtype, s);
    default: return launch_d<256, TP>(a, out_dtype, s);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, int part_dtype, int out_dtype,
                        hipStream_t s, const TimingHook& t) {
  hipError_t ev = record_event(t.start, s);
  const hipError_t e = part_dtype == SINK_ATTN_BF16   ? launch_tp<dev::bf16>(a, head_dim, out_dtype, s)
                       : part_dtype == SINK_ATTN_FP16 ? launch_tp<dev::f16>(a, head_dim, out_dtype, s)
                                                      : launch_tp<float>(a, head_dim, out_dtype, s);
  ev = first_error(ev, record_event(t.stop, s));
  return first_error(e, ev);
}

}  // namespace sinkattn
