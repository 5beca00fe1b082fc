// C ABI of libsinkattn.so, its host-only entry points: the tile schedule
// calls (argument checks, then the table built in schedule.cpp), status
// strings and the ABI version. No HIP call and no device code, so this file
// and schedule.cpp also build as plain C++ (the host sanitizer test does).
// Declarations and the contract are in include/sink_attn.h.
#include <cstdint>
#include <vector>

#include "sink_attn_internal.h"

using namespace sinkattn;

extern "C" {

sink_attn_status sink_attn_metadata(const sink_attn_problem* p,
                                    const int32_t* cu_seqlens_q_host,
                                    const int32_t* cu_seqlens_k_host,
                                    int32_t* meta_host,
                                    int64_t meta_capacity_words,
                                    int64_t* meta_words,
                                    int64_t* fwd_workspace_bytes,
                                    int64_t* bwd_workspace_bytes) {
  sink_attn_status st = validate_problem(p);
  if (st != SINK_ATTN_OK) return st;
  if (!meta_words || !fwd_workspace_bytes || !bwd_workspace_bytes)
    return SINK_ATTN_E_INVALID;
  if (p->layout_q != SINK_ATTN_TND) return SINK_ATTN_E_INVALID;
  st = validate_cu_seqlens(*p, cu_seqlens_q_host, cu_seqlens_k_host);
  if (st != SINK_ATTN_OK) return st;
  if (meta_host && meta_capacity_words < 0) return SINK_ATTN_E_INVALID;
  return build_metadata(*p, cu_seqlens_q_host, cu_seqlens_k_host, nullptr, 0, meta_host,
                        meta_capacity_words, meta_words, fwd_workspace_bytes,
                        bwd_workspace_bytes);
}

sink_attn_status sink_attn_metadata_padded(const sink_attn_problem* p,
                                           const int32_t* seqused_q_host,
                                           const int32_t* seqused_kv_host,
                                           int32_t* meta_host,
                                           int64_t meta_capacity_words,
                                           int64_t* meta_words,
                                           int64_t* fwd_workspace_bytes,
                                           int64_t* bwd_workspace_bytes) {
  sink_attn_status st = validate_problem(p);
  if (st != SINK_ATTN_OK) return st;
  if (!meta_words || !fwd_workspace_bytes || !bwd_workspace_bytes)
    return SINK_ATTN_E_INVALID;
  if (p->layout_q == SINK_ATTN_TND) return SINK_ATTN_E_INVALID;
  std::vector<int32_t> cu_q(static_cast<size_t>(p->batch) + 1);
  std::vector<int32_t> cu_k(static_cast<size_t>(p->batch) + 1);
  st = validate_seqused(*p, seqused_q_host, seqused_kv_host, cu_q.data(), cu_k.data());
  if (st != SINK_ATTN_OK) return st;
  if (meta_host && meta_capacity_words < 0) return SINK_ATTN_E_INVALID;
  const int mask = (seqused_q_host ? 1 : 0) | (seqused_kv_host ? 2 : 0);
  return build_metadata(*p, cu_q.data(), cu_k.data(), nullptr, mask, meta_host,
                        meta_capacity_words, meta_words, fwd_workspace_bytes,
                        bwd_workspace_bytes);
}

sink_attn_status sink_attn_metadata_paged(const sink_attn_problem* p,
                                          const sink_attn_paged_kv* kv,
                                          const int32_t* cu_seqlens_q_host,
                                          const int32_t* seqused_kv_host,
                                          const int32_t* block_table_host,
                                          int32_t* meta_host,
                                          int64_t meta_capacity_words,
                                          int64_t* meta_words,
                                          int64_t* fwd_workspace_bytes) {
  sink_attn_status st = validate_problem(p);
  if (st != SINK_ATTN_OK) return st;
  if (!meta_words || !fwd_workspace_bytes) return SINK_ATTN_E_INVALID;
  if (p->layout_q != SINK_ATTN_TND) return SINK_ATTN_E_INVALID;
  std::vector<int32_t> cu_k(static_cast<size_t>(p->batch) + 1);
  st = validate_paged(*p, kv, seqused_kv_host, block_table_host, cu_k.data());
  if (st != SINK_ATTN_OK) return st;
  st = validate_cu_seqlens(*p, cu_seqlens_q_host, cu_k.data());
  if (st != SINK_ATTN_OK) return st;
  if (p->dtype == SINK_ATTN_FP32) return SINK_ATTN_E_UNSUPPORTED;
  if (meta_host && meta_capacity_words < 0) return SINK_ATTN_E_INVALID;
  const PagedInfo info{*kv, block_table_host};
  int64_t bwd_bytes = 0;
  return build_metadata(*p, cu_seqlens_q_host, cu_k.data(), &info, 0, meta_host,
                        meta_capacity_words, meta_words, fwd_workspace_bytes, &bwd_bytes);
}

const char* sink_attn_status_string(sink_attn_status s) {
  switch (s) {
    case SINK_ATTN_OK: return "ok";
    case SINK_ATTN_E_INVALID: return "invalid argument";
    case SINK_ATTN_E_UNSUPPORTED: return "unsupported head_dim, dtype or shape";
    case SINK_ATTN_E_META_MISMATCH: return "metadata does not match the call";
    case SINK_ATTN_E_BUFFER_TOO_SMALL: return "buffer too small";
    case SINK_ATTN_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t sink_attn_abi_version(void) { return SINK_ATTN_ABI_VERSION; }

}  // extern "C"
