// fp32 path: the same method at full fp32 precision with plain VALU
// arithmetic, one thread per (row, head). It serves fp32 problems, which are
// small and latency-bound (the bf16 MFMA kernels are the throughput path).
//
// Forward: online softmax over the row's kept key interval, seeded with the
// sink ("CANN ops-transformer: flash_attn", Formula section: m = max(sink,
// max S), the sink term e^(sink - m) in the denominator). Backward: the
// chain rule through softmax([S, sink]) ("slime: learnable_softmax_
// attention.py", backward): dS = P (dP - D), P = e^(S - lse) with the
// sink-inclusive lse; dQ per query row, dK/dV per key over the query rows
// of every q-head of the GQA group.
#include "bwd_common.h"

namespace sinkattn {
namespace {

using namespace dev;

template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(FwdArgs a) {
  const int row = blockIdx.x * 128 + threadIdx.x;
  if (row >= a.total_q * a.hq) return;
  const int t = row / a.hq, h = row % a.hq, hk = h / a.group;
  int b, i;
  q_row_of(a, t, b, i);
  const int lq = q_len(a, b);
  if (i >= lq) return;   // padding row of a padded layout
  const int k0 = k_start(a, b), lk = k_len(a, b);
  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);
  const int64_t off = (int64_t)(t - i) * a.g.q_seq + (int64_t)i * a.g.q_row + h * a.g.q_head;
  const float* qp = static_cast<const float*>(a.q) + off;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = qp[d] * a.scale * kLog2e; o[d] = 0.f; }
  const float sink = a.sinks ? a.sinks[h] : kNegInf;
  float m = sink * kLog2e;
  float l = sink > kNegInf ? 1.f : 0.f;
  for (int jj = jlo; jj <= jhi; ++jj) {
    const int64_t ko = (int64_t)k0 * a.g.k_seq + (int64_t)jj * a.g.k_row + hk * a.g.k_head;
    const float* kp = static_cast<const float*>(a.k) + ko;
    const float* vp = static_cast<const float*>(a.v) + ko;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], kp[d], s);
    const float mn = fmaxf(m, s);
    const float alpha = exp2_hw(m - mn);
    const float p = exp2_hw(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(o[d], alpha, p * vp[d]);
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = static_cast<float*>(a.out) + (int64_t)(t - i) * a.g.o_seq + (int64_t)i * a.g.o_row +
              h * a.g.o_head;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  a.lse[(int64_t)(t - i) * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head] =
      l > 0.f ? (m + log2_hw(l)) * kLn2 : kNegInf;
}

template <int D>
__global__ __launch_bounds__(128) void bwd_dq_f32_kernel(BwdArgs a) {
  const int row = blockIdx.x * 128 + threadIdx.x;
  if (row >= a.total_q * a.hq) return;
  const int t = row / a.hq, h = row % a.hq, hk = h / a.group;
  int b, i;
  q_row_of(a, t, b, i);
  const int lq = q_len(a, b);
  if (i >= lq) return;
  const int k0 = k_start(a, b), lk = k_len(a, b);
  int jlo, jhi;
  row_key_range(i, lq, lk, a.causal, a.win_left, a.win_right, jlo, jhi);
  const int64_t off = (int64_t)(t - i) * a.g.q_seq + (int64_t)i * a.g.q_row + h * a.g.q_head;
  const float* qp = static_cast<const float*>(a.q) + off;
  const float* dop = static_cast<const float*>(a.dout) + (int64_t)(t - i) * a.g.o_seq +
                     (int64_t)i * a.g.o_row + h * a.g.o_head;
  float q[D], g[D], dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = qp[d]; g[d] = dop[d]; dq[d] = 0.f; }
  const float lse2 =
      a.lse[(int64_t)(t - i) * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head] * kLog2e;
  const float Dt = a.dval[(int64_t)h * a.total_q + t];
  const float c2 = a.scale * kLog2e;
  for (int jj = jlo; jj <= jhi; ++jj) {
    const int64_t ko = (int64_t)k0 * a.g.k_seq + (int64_t)jj * a.g.k_row + hk * a.g.k_head;
    const float* kp = static_cast<const float*>(a.k) + ko;
    const float* vp = static_cast<const float*>(a.v) + ko;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) { s = __builtin_fmaf(q[d], kp[d], s); dp = __builtin_fmaf(g[d], vp[d], dp); }
    const float p = exp2_hw(__builtin_fmaf(s, c2, -lse2));
    const float ds = a.scale * p * (dp - Dt);
#pragma unroll
    for (int d = 0; d < D; ++d) dq[d] = __builtin_fmaf(ds, kp[d], dq[d]);
  }
  float* dqp = static_cast<float*>(a.dq) + off;
#pragma unroll
  for (int d = 0; d < D; ++d) dqp[d] = dq[d];
}

template <int D>
__global__ __launch_bounds__(128) void bwd_dkdv_f32_kernel(BwdArgs a) {
  const int row = blockIdx.x * 128 + threadIdx.x;
  if (row >= a.total_k * a.hk) return;
  const int t = row / a.hk, hk = row % a.hk;
  int b, j;
  k_row_of(a, t, b, j);
  const int lk = k_len(a, b);
  if (j >= lk) return;   // padding key of a padded layout
  const int q0 = q_start(a, b), lq = q_len(a, b);
  int ilo, ihi;
  key_row_range(j, lq, lk, a.causal, a.win_left, a.win_right, ilo, ihi);
  const int64_t off = (int64_t)(t - j) * a.g.k_seq + (int64_t)j * a.g.k_row + hk * a.g.k_head;
  const float* kp = static_cast<const float*>(a.k) + off;
  const float* vp = static_cast<const float*>(a.v) + off;
  float kk[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { kk[d] = kp[d]; vv[d] = vp[d]; dk[d] = 0.f; dv[d] = 0.f; }
  const float c2 = a.scale * kLog2e;
  for (int g = 0; g < a.group; ++g) {
    const int h = hk * a.group + g;
    for (int i = ilo; i <= ihi; ++i) {
      const int64_t qo = (int64_t)q0 * a.g.q_seq + (int64_t)i * a.g.q_row + h * a.g.q_head;
      const float* qp = static_cast<const float*>(a.q) + qo;
      const float* dop = static_cast<const float*>(a.dout) + (int64_t)q0 * a.g.o_seq +
                         (int64_t)i * a.g.o_row + h * a.g.o_head;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) { s = __builtin_fmaf(qp[d], kk[d], s); dp = __builtin_fmaf(dop[d], vv[d], dp); }
      const float lse2 =
          a.lse[(int64_t)q0 * a.g.l_seq + (int64_t)i * a.g.l_row + h * a.g.l_head] * kLog2e;
      const float p = exp2_hw(__builtin_fmaf(s, c2, -lse2));
      const float ds = a.scale * p * (dp - a.dval[(int64_t)h * a.total_q + q0 + i]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(p, dop[d], dv[d]);
        dk[d] = __builtin_fmaf(ds, qp[d], dk[d]);
      }
    }
  }
  float* dkp = static_cast<float*>(a.dk) + off;
  float* dvp = static_cast<float*>(a.dv) + off;
#pragma unroll
  for (int d = 0; d < D; ++d) { dkp[d] = dk[d]; dvp[d] = dv[d]; }
}

template <int D>
hipError_t launch_fwd_f32_d(const FwdArgs& a, hipStream_t s, const TimingHook& th) {
  const int rows = a.total_q * a.hq;
  hipError_t ev = record_event(th.start, s);
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((rows + 127) / 128), dim3(128), 0, s, a);
  ev = first_error(ev, record_event(th.stop, s));
  return first_error(hipGetLastError(), ev);
}

template <int D>
hipError_t launch_bwd_f32_d(const BwdArgs& a, hipStream_t s, const TimingHook& th) {
  hipError_t e = launch_bwd_pre<D, float>(a, s);
  if (e != hipSuccess) return e;
  const int rq = a.total_q * a.hq, rk = a.total_k * a.hk;
  hipError_t ev = record_event(th.start, s);
  hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3((rq + 127) / 128), dim3(128), 0, s, a);
  hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3((rk + 127) / 128), dim3(128), 0, s, a);
  ev = first_error(ev, record_event(th.stop, s));
  e = first_error(hipGetLastError(), ev);
  if (e != hipSuccess) return e;
  return launch_dsink_finalize(a, s);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, hipStream_t s, const TimingHook& t) {
  return head_dim == 128 ? launch_fwd_f32_d<128>(a, s, t) : launch_fwd_f32_d<64>(a, s, t);
}

hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, hipStream_t s, const TimingHook& t) {
  return head_dim == 128 ? launch_bwd_f32_d<128>(a, s, t) : launch_bwd_f32_d<64>(a, s, t);
}

}  // namespace sinkattn
