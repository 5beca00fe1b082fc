// C ABI of libsinkattn.so, the entry points that run on the GPU: argument
// checks, workspace carving and kernel dispatch (the host-only ones are in
// metadata.cpp). Declarations and the contract are in include/sink_attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "sink_attn_internal.h"

using namespace sinkattn;

// Scratch of sink_attn_bwd_noalloc: one copy per GPU, held until the
// process ends. Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[SINK_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` per device id, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

thread_local TimingHook g_timing;

TimingHook take_timing() {
  TimingHook t = g_timing;
  g_timing = TimingHook{};
  return t;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int64_t header_i64(const int32_t* h, int lo, int hi) {
  return static_cast<int64_t>(static_cast<uint32_t>(h[lo])) |
         (static_cast<int64_t>(h[hi]) << 32);
}

sink_attn_status common_checks(const sink_attn_problem* p,
                               const int32_t* meta_host,
                               const int32_t* meta_dev, float scale,
                               const sink_attn_paged_kv* kv = nullptr) {
  sink_attn_status st = validate_problem(p);
  if (st != SINK_ATTN_OK) return st;
  if (!meta_host || !meta_dev) return SINK_ATTN_E_INVALID;
  if (!std::isfinite(scale) || !(scale > 0.f)) return SINK_ATTN_E_INVALID;
  return check_header(*p, meta_host, kv);
}

// Table upload: each thread moves 16 bytes (or 4 in the ragged tail) from
// the pinned host table, read by the GPU through its device address.
__global__ __launch_bounds__(256) void upload_table_kernel(const int32_t* __restrict__ src,
                                                           int32_t* __restrict__ dst,
                                                           int64_t words) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= words) {
    *reinterpret_cast<int4*>(dst + i) = *reinterpret_cast<const int4*>(src + i);
  } else {
    for (int64_t j = i; j < words; ++j) dst[j] = src[j];
  }
}

// Window bound handed to the kernels. A window of max_seqlen_q +
// max_seqlen_k or more never excludes a key (the bottom-right aligned row
// position lies in [-max_seqlen_q, max_seqlen_k)), so it is passed on as
// unbounded (-1): the kernels' 32-bit mask arithmetic then stays within
// +-2^30 (validate_problem bounds every sequence below 2^28 rows).
int kernel_window(int32_t w, const sink_attn_problem* p) {
  if (w < 0) return -1;
  return static_cast<int64_t>(w) >= static_cast<int64_t>(p->max_seqlen_q) + p->max_seqlen_k
             ? -1 : w;
}

FwdArgs fwd_args(const sink_attn_problem* p, const void* q, const void* k,
                 const void* v, const int32_t* cu_q, const int32_t* cu_k,
                 const int32_t* used_q, const int32_t* used_k,
                 const float* sinks, float scale, void* out, float* lse) {
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.cu_q = cu_q; a.cu_k = cu_k;
  a.g = make_geometry(*p, used_q, used_k);
  a.sinks = sinks;
  a.out = out; a.lse = lse;
  a.batch = p->batch; a.hq = p->num_heads_q; a.hk = p->num_heads_k;
  a.group = p->num_heads_q / p->num_heads_k;
  a.causal = p->causal;
  a.win_left = kernel_window(p->win_left, p);
  a.win_right = kernel_window(p->win_right, p);
  a.total_q = p->total_q; a.total_k = p->total_k;
  a.scale = scale;
  return a;
}

// Split-KV items, per-sequence table and partials workspace of a decode-mode
// table.
bool decode_args(FwdArgs& a, const sink_attn_problem* p, const int32_t* meta_host,
                 const int32_t* meta_dev, void* workspace) {
  const FwdWorkspace w = fwd_workspace_layout(meta_host[kDecRows], p->head_dim,
                                              p->dtype, kModeDecode);
  // the partials must fit the workspace the header asked the caller for
  if (w.bytes > header_i64(meta_host, kFwdWsLo, kFwdWsHi) || (w.bytes > 0 && !workspace))
    return false;
  char* base = static_cast<char*>(workspace);
  a.items = meta_dev + meta_host[kDecOff];
  a.n_items = meta_host[kNDec];
  a.dec_seq = meta_dev + meta_host[kDecSeqOff];
  a.ws_o = reinterpret_cast<float*>(base + w.o_off);
  a.ws_m = reinterpret_cast<float*>(base + w.m_off);
  a.ws_l = reinterpret_cast<float*>(base + w.l_off);
  return true;
}

// The packed calls take TND problems with cu_seqlens; the padded calls take
// BSND / BNSD problems whose seqused pointers are null exactly where they
// were for the metadata. Called after common_checks.
sink_attn_status check_family(const sink_attn_problem* p, const int32_t* meta_host,
                              bool padded, const int32_t* used_q, const int32_t* used_k) {
  if ((p->layout_q != SINK_ATTN_TND) != padded) return SINK_ATTN_E_INVALID;
  const int mask = (used_q ? 1 : 0) | (used_k ? 2 : 0);
  if (meta_host[kUsedMask] != mask) return SINK_ATTN_E_META_MISMATCH;
  return SINK_ATTN_OK;
}

sink_attn_status fwd_impl(const sink_attn_problem* p, const int32_t* meta_host,
                          const int32_t* meta_dev, const void* q, const void* k,
                          const void* v, const int32_t* cu_q, const int32_t* cu_k,
                          const int32_t* used_q, const int32_t* used_k,
                          const float* sink_logits, float scale, void* out, float* lse,
                          void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse) return SINK_ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(lse))
    return SINK_ATTN_E_INVALID;
  const int64_t need = header_i64(meta_host, kFwdWsLo, kFwdWsHi);
  if (workspace_bytes < need) return SINK_ATTN_E_BUFFER_TOO_SMALL;
  if (need > 0 && (!workspace || !aligned16(workspace))) return SINK_ATTN_E_INVALID;

  const int mode = meta_host[kMode];
  FwdArgs a = fwd_args(p, q, k, v, cu_q, cu_k, used_q, used_k, sink_logits, scale, out, lse);
  const TimingHook t = take_timing();
  hipError_t e;
  if (p->dtype == SINK_ATTN_FP32) {
    e = launch_fwd_f32(a, p->head_dim, stream, t);
  } else if (mode == kModeDecode) {
    if (!decode_args(a, p, meta_host, meta_dev, workspace)) return SINK_ATTN_E_META_MISMATCH;
    e = launch_fwd_16(a, p->head_dim, p->dtype, mode, stream, t);
  } else {
    a.items = meta_dev + meta_host[kFwdOff];
    a.n_items = meta_host[kNFwd];
    e = launch_fwd_16(a, p->head_dim, p->dtype, mode, stream, t);
  }
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_E_HIP;
}

sink_attn_status bwd_impl(const sink_attn_problem* p, const int32_t* meta_host,
                          const int32_t* meta_dev, const void* dout, const void* q,
                          const void* k, const void* v, const void* out, const float* lse,
                          const int32_t* cu_q, const int32_t* cu_k,
                          const int32_t* used_q, const int32_t* used_k,
                          const float* sink_logits, float scale, void* dq, void* dk,
                          void* dv, float* dsink, void* workspace,
                          int64_t workspace_bytes, hipStream_t stream) {
  if (!dout || !q || !k || !v || !out || !lse || !dq || !dk || !dv)
    return SINK_ATTN_E_INVALID;
  if ((sink_logits == nullptr) != (dsink == nullptr)) return SINK_ATTN_E_INVALID;
  if (!aligned16(dout) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(out) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return SINK_ATTN_E_INVALID;
  const int64_t need = header_i64(meta_host, kBwdWsLo, kBwdWsHi);
  if (workspace_bytes < need) return SINK_ATTN_E_BUFFER_TOO_SMALL;
  if (need > 0 && (!workspace || !aligned16(workspace))) return SINK_ATTN_E_INVALID;

  const int64_t pre_blocks = meta_host[kBwdPreBlocks];
  const BwdWorkspace w = bwd_workspace_layout(p->total_q, p->num_heads_q,
                                              p->head_dim, p->dtype, pre_blocks);
  char* base = static_cast<char*>(workspace);
  BwdArgs a{};
  a.dout = dout; a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.cu_q = cu_q; a.cu_k = cu_k; a.sinks = sink_logits;
  a.g = make_geometry(*p, used_q, used_k);
  a.dq = dq; a.dk = dk; a.dv = dv; a.dsink = dsink;
  a.items = meta_dev + meta_host[kBwdOff];
  a.n_items = meta_host[kNBwd];
  a.items_q = meta_dev + meta_host[kFwdOff];
  a.n_items_q = meta_host[kNFwd];
  a.pre_blocks = static_cast<int>(pre_blocks);
  a.dval = reinterpret_cast<float*>(base + w.dval_off);
  a.part = reinterpret_cast<float*>(base + w.part_off);
  a.batch = p->batch; a.hq = p->num_heads_q; a.hk = p->num_heads_k;
  a.group = p->num_heads_q / p->num_heads_k;
  a.causal = p->causal;
  a.win_left = kernel_window(p->win_left, p);
  a.win_right = kernel_window(p->win_right, p);
  a.total_q = p->total_q; a.total_k = p->total_k;
  a.scale = scale;
  const TimingHook t = take_timing();
  hipError_t e = p->dtype == SINK_ATTN_FP32
                     ? launch_bwd_f32(a, p->head_dim, stream, t)
                     : launch_bwd_16(a, p->head_dim, p->dtype, stream, t);
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_E_HIP;
}

}  // namespace

extern "C" {

sink_attn_status sink_attn_fwd(const sink_attn_problem* p,
                               const int32_t* meta_host,
                               const int32_t* meta_dev, const void* q,
                               const void* k, const void* v,
                               const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k,
                               const float* sink_logits, float scale,
                               void* out, float* lse, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, false, nullptr, nullptr);
  if (st != SINK_ATTN_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return SINK_ATTN_E_INVALID;
  return fwd_impl(p, meta_host, meta_dev, q, k, v, cu_seqlens_q, cu_seqlens_k, nullptr,
                  nullptr, sink_logits, scale, out, lse, workspace, workspace_bytes, stream);
}

sink_attn_status sink_attn_fwd_padded(const sink_attn_problem* p,
                                      const int32_t* meta_host,
                                      const int32_t* meta_dev, const void* q,
                                      const void* k, const void* v,
                                      const int32_t* seqused_q,
                                      const int32_t* seqused_kv,
                                      const float* sink_logits, float scale,
                                      void* out, float* lse, void* workspace,
                                      int64_t workspace_bytes, hipStream_t stream) {
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, true, seqused_q, seqused_kv);
  if (st != SINK_ATTN_OK) return st;
  return fwd_impl(p, meta_host, meta_dev, q, k, v, nullptr, nullptr, seqused_q, seqused_kv,
                  sink_logits, scale, out, lse, workspace, workspace_bytes, stream);
}

sink_attn_status sink_attn_fwd_paged(const sink_attn_problem* p,
                                     const sink_attn_paged_kv* kv,
                                     const int32_t* meta_host,
                                     const int32_t* meta_dev, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_table,
                                     const int32_t* cu_seqlens_q,
                                     const int32_t* seqused_kv,
                                     const float* sink_logits, float scale,
                                     void* out, float* lse, void* workspace,
                                     int64_t workspace_bytes,
                                     hipStream_t stream) {
  if (!kv) return SINK_ATTN_E_INVALID;
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale, kv);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, false, nullptr, nullptr);
  if (st != SINK_ATTN_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !out || !lse || !cu_seqlens_q ||
      !seqused_kv)
    return SINK_ATTN_E_INVALID;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(block_table))
    return SINK_ATTN_E_INVALID;
  const int64_t need = header_i64(meta_host, kFwdWsLo, kFwdWsHi);
  if (workspace_bytes < need) return SINK_ATTN_E_BUFFER_TOO_SMALL;
  if (need > 0 && (!workspace || !aligned16(workspace))) return SINK_ATTN_E_INVALID;
  const int mode = meta_host[kMode];

  FwdArgs a = fwd_args(p, q, k_cache, v_cache, cu_seqlens_q, nullptr, nullptr, nullptr,
                       sink_logits, scale, out, lse);
  if (mode == kModeDecode) {
    if (!decode_args(a, p, meta_host, meta_dev, workspace)) return SINK_ATTN_E_META_MISMATCH;
  } else {
    a.items = meta_dev + meta_host[kFwdOff];
    a.n_items = meta_host[kNFwd];
  }
  a.block_table = block_table;
  a.seqused_k = seqused_kv;
  a.page_size = kv->block_size;
  a.page_cols = kv->max_blocks_per_seq;
  a.page_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + kv->block_size - 1) /
                                       static_cast<uint64_t>(kv->block_size));
  const int64_t bs = kv->block_size, hkn = p->num_heads_k, d = p->head_dim;
  a.page_stride = bs * hkn * d;
  if (kv->layout == SINK_ATTN_PA_BNBD) { a.page_row = d; a.page_head = bs * d; }
  else { a.page_row = hkn * d; a.page_head = d; }
  const TimingHook t = take_timing();
  const hipError_t e = launch_fwd_16(a, p->head_dim, p->dtype, mode, stream, t);
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_E_HIP;
}

sink_attn_status sink_attn_bwd(const sink_attn_problem* p,
                               const int32_t* meta_host,
                               const int32_t* meta_dev, const void* dout,
                               const void* q, const void* k, const void* v,
                               const void* out, const float* lse,
                               const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k,
                               const float* sink_logits, float scale, void* dq,
                               void* dk, void* dv, float* dsink,
                               void* workspace, int64_t workspace_bytes,
                               hipStream_t stream) {
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, false, nullptr, nullptr);
  if (st != SINK_ATTN_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return SINK_ATTN_E_INVALID;
  return bwd_impl(p, meta_host, meta_dev, dout, q, k, v, out, lse, cu_seqlens_q,
                  cu_seqlens_k, nullptr, nullptr, sink_logits, scale, dq, dk, dv, dsink,
                  workspace, workspace_bytes, stream);
}

sink_attn_status sink_attn_bwd_noalloc(const sink_attn_problem* p,
                                       const int32_t* meta_host,
                                       const int32_t* meta_dev, const void* dout,
                                       const void* q, const void* k, const void* v,
                                       const void* out, const float* lse,
                                       const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k,
                                       const float* sink_logits, float scale, void* dq,
                                       void* dk, void* dv, float* dsink,
                                       hipStream_t stream) {
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, false, nullptr, nullptr);
  if (st != SINK_ATTN_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return SINK_ATTN_E_INVALID;
  if (header_i64(meta_host, kBwdWsLo, kBwdWsHi) > SINK_ATTN_NOALLOC_SCRATCH_BYTES)
    return SINK_ATTN_E_BUFFER_TOO_SMALL;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return SINK_ATTN_E_HIP;
  return bwd_impl(p, meta_host, meta_dev, dout, q, k, v, out, lse, cu_seqlens_q,
                  cu_seqlens_k, nullptr, nullptr, sink_logits, scale, dq, dk, dv, dsink, ws,
                  SINK_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

sink_attn_status sink_attn_bwd_padded(const sink_attn_problem* p,
                                      const int32_t* meta_host,
                                      const int32_t* meta_dev, const void* dout,
                                      const void* q, const void* k, const void* v,
                                      const void* out, const float* lse,
                                      const int32_t* seqused_q,
                                      const int32_t* seqused_kv,
                                      const float* sink_logits, float scale, void* dq,
                                      void* dk, void* dv, float* dsink,
                                      void* workspace, int64_t workspace_bytes,
                                      hipStream_t stream) {
  sink_attn_status st = common_checks(p, meta_host, meta_dev, scale);
  if (st != SINK_ATTN_OK) return st;
  st = check_family(p, meta_host, true, seqused_q, seqused_kv);
  if (st != SINK_ATTN_OK) return st;
  return bwd_impl(p, meta_host, meta_dev, dout, q, k, v, out, lse, nullptr, nullptr,
                  seqused_q, seqused_kv, sink_logits, scale, dq, dk, dv, dsink, workspace,
                  workspace_bytes, stream);
}

sink_attn_status sink_attn_merge(int32_t num_parts, int32_t total_q,
                                 int32_t num_heads_q, int32_t head_dim,
                                 int32_t part_dtype, int32_t out_dtype,
                                 const void* partial_out, const float* partial_lse,
                                 const float* sink_logits, void* out, float* lse,
                                 hipStream_t stream) {
  if (num_parts <= 0 || num_parts > kMaxMergeParts || total_q <= 0 || num_heads_q <= 0)
    return SINK_ATTN_E_INVALID;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return SINK_ATTN_E_UNSUPPORTED;
  const auto known = [](int32_t d) {
    return d == SINK_ATTN_FP32 || d == SINK_ATTN_BF16 || d == SINK_ATTN_FP16;
  };
  if (!known(part_dtype) || !known(out_dtype)) return SINK_ATTN_E_UNSUPPORTED;
  if (!partial_out || !partial_lse || !out || !lse) return SINK_ATTN_E_INVALID;
  if (!aligned16(partial_out) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(partial_lse) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return SINK_ATTN_E_INVALID;
  // the widest index: parts x rows x head_dim elements
  if (static_cast<int64_t>(num_parts) * total_q * num_heads_q * head_dim >= (int64_t(1) << 40))
    return SINK_ATTN_E_UNSUPPORTED;
  MergeArgs a{};
  a.part_out = partial_out; a.part_lse = partial_lse; a.sinks = sink_logits;
  a.out = out; a.lse = lse;
  a.parts = num_parts; a.total_q = total_q; a.hq = num_heads_q;
  const TimingHook t = take_timing();
  const hipError_t e = launch_merge(a, head_dim, part_dtype, out_dtype, stream, t);
  return e == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_E_HIP;
}

sink_attn_status sink_attn_upload_table(const int32_t* host, int32_t* dev, int64_t words,
                                        hipStream_t stream) {
  if (!host || !dev || words < 0) return SINK_ATTN_E_INVALID;
  if (words == 0) return SINK_ATTN_OK;
  // 16-byte moves need both ends 16-byte aligned (pinned and device
  // allocations are)
  if (!aligned16(host) || !aligned16(dev)) return SINK_ATTN_E_INVALID;
  hipPointerAttribute_t ha{}, da{};
  if (hipPointerGetAttributes(&ha, host) != hipSuccess || ha.type != hipMemoryTypeHost ||
      !ha.devicePointer) {
    (void)hipGetLastError();                    // clear a lookup failure
    return SINK_ATTN_E_INVALID;
  }
  if (hipPointerGetAttributes(&da, dev) != hipSuccess || da.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return SINK_ATTN_E_INVALID;
  }
  const char* h0 = reinterpret_cast<const char*>(host);
  const char* d0 = reinterpret_cast<const char*>(dev);
  const int64_t bytes = words * 4;
  if (h0 < d0 + bytes && d0 < h0 + bytes) return SINK_ATTN_E_INVALID;
  const int64_t threads = (words + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > INT32_MAX) return SINK_ATTN_E_INVALID;
  hipLaunchKernelGGL(upload_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, static_cast<const int32_t*>(ha.devicePointer), dev, words);
  return hipGetLastError() == hipSuccess ? SINK_ATTN_OK : SINK_ATTN_E_HIP;
}

sink_attn_status sink_attn_arm_timing(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return SINK_ATTN_E_INVALID;
  g_timing.start = start;
  g_timing.stop = stop;
  return SINK_ATTN_OK;
}

}  // extern "C"
