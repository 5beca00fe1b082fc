// Internal declarations shared by the host scheduler, the C ABI layer and
// the kernel launchers of libsinkattn.so.
#pragma once

#include <cstdint>
#include <hip/hip_runtime_api.h>

#include "sink_attn.h"

namespace sinkattn {

// ---------------------------------------------------------------------------
// Metadata table: kHeaderWords int32 header words, then the item arrays.
// ---------------------------------------------------------------------------
enum MetaWord : int {
  kMagic = 0, kVersion, kBatch, kHq, kHk, kHeadDim, kTq, kTk, kMaxQ, kMaxK,
  kCausal, kWinL, kWinR, kDtype, kMode,
  kWordFwdBM, kWordFwdBN, kWordBwdBM, kWordBwdBN, kWordDecBN, kWordDecChunk,
  kNFwd, kFwdOff, kNBwd, kBwdOff, kNDec, kDecOff, kDecSeqOff, kDecRows,
  kFwdWsLo, kFwdWsHi, kBwdWsLo, kBwdWsHi, kCuHash, kMetaWords,
  kBwdPreBlocks,
  kPaged, kPageSize, kPageMaxBlocks, kPageNumBlocks, kPageHash,
  kLayoutQ, kLayoutOut, kSeqQ, kSeqK, kUsedMask, kPageLayout,
  kFwdWords,           // the forward reads words [0, kFwdWords) of the table
  kWordDecTail,        // split-KV chunk of the sequences at the end of the grid
  kWordDecTailPct,     // share (percent) of the span length cut into those
  kHeaderWords = 56
};
static_assert(kFwdWords == SINK_ATTN_META_FWD_WORDS, "header word of the forward prefix");

constexpr int32_t kMagicValue = 0x4B4E4953;  // "SINK" little-endian
constexpr int kItemWords = 16;

// Table order: header, decode items, decode per-sequence table, forward
// items, backward items. The forward reads the header and, in decode mode,
// the decode items and per-sequence table, else the forward items: a
// prefix of the table.
// Forward item:  b, qt, kt_lo, kt_hi, kf_lo, kf_hi, 0, 0
// Backward item: b, kt, qt_lo, qt_hi, qf_lo, qf_hi, 0, 0
// Decode item:   b, split, k_lo, k_hi, row_base, 0, 0, 0
// Words 8-11 of every item: the sequence's first query row and query row
// count, first key row and key row count (as q_start, q_len, k_start,
// k_len give them; first key row 0 for a paged cache), so that a block has
// them with its item instead of one memory latency later; 12-15 unused.
// Decode per-sequence table (2 words per sequence): first item, count.

enum Mode : int32_t { kModePrefill = 0, kModeDecode = 1 };

// Tile shapes of the bf16 kernels (recorded in the header; the kernels are
// compiled for exactly these values and the ABI layer checks them).
constexpr int kFwdBM = 128;    // query rows per forward work item (4 waves x 32)
constexpr int kFwdBN = 64;     // keys per forward tile step
constexpr int kBwdBM = 64;     // query rows per backward tile step (D <= 128)
// Query rows per backward tile step of a head dim: 32 at D = 256, where
// five [64 x 256] tiles would not fit the LDS of the dK/dV kernel.
constexpr int bwd_tile_rows(int head_dim) { return head_dim > 128 ? 32 : kBwdBM; }
constexpr int kBwdBN = 128;    // keys per backward work item (2 halves of 64)
constexpr int kDecBN = 64;     // keys per split-KV tile step
constexpr int kDecChunk = 4096;// keys per split-KV work item (at most)
constexpr int kDecMinChunk = 512;      // shortest chunk, for grids too small to fill the chip
constexpr int kDecMinBlocks = 512;     // split-KV blocks a grid should reach (one per slot)
constexpr int kDecTailChunk = 1024;    // chunk of the sequences at the end of a long grid
constexpr int kDecTailPercent = 10;    // share of the span length cut that way
constexpr int kDecMaxRows = 64;// (query rows x GQA group) handled per split item
constexpr int kPreRows = 64;   // tokens per block of the backward preprocess
constexpr int kMaxMergeParts = 4096;  // partials one context-parallel merge accepts

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Workspace layouts (byte offsets), derived from the header only.
struct FwdWorkspace {
  int64_t o_off, m_off, l_off, bytes;
};
struct BwdWorkspace {
  int64_t dval_off, part_off, bytes;
};
FwdWorkspace fwd_workspace_layout(int64_t dec_rows, int head_dim, int dtype,
                                  int mode);
BwdWorkspace bwd_workspace_layout(int64_t total_q, int hq, int head_dim,
                                  int dtype, int64_t pre_blocks);

// Paged K/V as seen by the schedule builder: the sizes and the host block
// table (hashed into the header).
struct PagedInfo {
  sink_attn_paged_kv kv;
  const int32_t* block_table;
};

// Host checks and the schedule builder (schedule.cpp).
sink_attn_status validate_problem(const sink_attn_problem* p);
sink_attn_status validate_cu_seqlens(const sink_attn_problem& p,
                                     const int32_t* cu_q, const int32_t* cu_k);
// Padded layouts: checks the host used lengths (null: all S) and writes
// their prefix sums (batch + 1 words each), which is all the schedule needs.
sink_attn_status validate_seqused(const sink_attn_problem& p, const int32_t* used_q,
                                  const int32_t* used_k, int32_t* cu_q_out,
                                  int32_t* cu_k_out);
// Checks a paged layout against the problem and the host tables, and
// writes the key-length prefix sums (batch + 1 words) into cu_k_out.
sink_attn_status validate_paged(const sink_attn_problem& p,
                                const sink_attn_paged_kv* kv,
                                const int32_t* seqused_kv,
                                const int32_t* block_table, int32_t* cu_k_out);
// Builds the table; writes it when `out` is non-null and capacity allows.
// `paged` is null for contiguous keys and values; `used_mask` records which
// seqused arrays a padded-layout call passes (1: q, 2: kv).
sink_attn_status build_metadata(const sink_attn_problem& p, const int32_t* cu_q,
                                const int32_t* cu_k, const PagedInfo* paged,
                                int used_mask, int32_t* out, int64_t capacity,
                                int64_t* words, int64_t* fwd_ws, int64_t* bwd_ws);
// Header against the call; `kv` is null for the contiguous calls.
sink_attn_status check_header(const sink_attn_problem& p, const int32_t* meta,
                              const sink_attn_paged_kv* kv);

// ---------------------------------------------------------------------------
// Kernel arguments and launchers (kernels_*.hip).
// ---------------------------------------------------------------------------
// Where the rows of every sequence live. Sequence b holds rows
// [0, len(b)) starting at row start(b) of its tensors: TND takes both from
// cu_seqlens; the padded layouts (BSND, BNSD) have start(b) = b * seq and
// len(b) = used[b] (or seq). Row i of head h of sequence b sits at element
//   start(b) * x_seq + i * x_row + h * x_head
// of q/dq (x = q), out/dout (x = o), k/v/dk/dv (x = k) and lse (x = l).
struct Geometry {
  const int32_t* used_q;    // padded layouts: rows in use (null: all seq_q)
  const int32_t* used_k;
  int seq_q, seq_k;         // padded layouts: rows per batch entry; TND: 0
  int64_t q_seq, q_row, q_head;
  int64_t o_seq, o_row, o_head;
  int64_t k_seq, k_row, k_head;
  int64_t l_seq, l_row, l_head;
};
// The geometry of a problem's layout (TND: the contiguous THD tensors and
// the [Hq, Tq] lse).
Geometry make_geometry(const sink_attn_problem& p, const int32_t* used_q,
                       const int32_t* used_k);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  Geometry g;
  const float* sinks;       // null: no sink
  void* out;
  float* lse;
  const int32_t* items;     // device: forward or decode items
  const int32_t* dec_seq;   // device: decode per-sequence table
  float* ws_o;              // decode partials
  float* ws_m;
  float* ws_l;
  // paged K/V (split-KV path only); k, v are then the caches
  const int32_t* block_table;
  const int32_t* seqused_k;
  int page_size, page_cols;  // block_size, max_blocks_per_seq
  uint32_t page_magic;       // ceil(2^32 / block_size)
  // element offset of (page p, slot s, kv-head h): p*page_stride + s*page_row + h*page_head
  int64_t page_stride, page_row, page_head;
  int n_items;
  int batch, hq, hk, group, causal, win_left, win_right;
  int total_q, total_k;
  float scale;
};

struct BwdArgs {
  const void* dout;
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  Geometry g;
  const float* sinks;
  void* dq;
  void* dk;
  void* dv;
  float* dsink;
  const int32_t* items;     // device: backward (key tile) items
  const int32_t* items_q;   // device: forward (query tile) items, for dQ
  float* dval;              // [hq, total_q]
  float* part;              // [hq, pre_blocks]
  int n_items, n_items_q, pre_blocks;
  int batch, hq, hk, group, causal, win_left, win_right;
  int total_q, total_k;
  float scale;
};

struct MergeArgs {
  const void* part_out;     // [parts, total_q, hq, D]
  const float* part_lse;    // [parts, hq, total_q], sink-free
  const float* sinks;       // null: no sink
  void* out;
  float* lse;
  int parts, total_q, hq;
};

struct TimingHook {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Records `e` on `s` when a timing event was armed; the launchers fold the
// status into their own.
inline hipError_t record_event(hipEvent_t e, hipStream_t s) {
  return e ? hipEventRecord(e, s) : hipSuccess;
}
// The first failure of two calls made in that order.
inline hipError_t first_error(hipError_t a, hipError_t b) { return a != hipSuccess ? a : b; }

// 16-bit inputs (dtype SINK_ATTN_BF16 or SINK_ATTN_FP16), MFMA kernels
hipError_t launch_fwd_16(const FwdArgs& a, int head_dim, int dtype, int mode,
                         hipStream_t s, const TimingHook& t);
hipError_t launch_bwd_16(const BwdArgs& a, int head_dim, int dtype, hipStream_t s,
                         const TimingHook& t);
hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, hipStream_t s,
                          const TimingHook& t);
hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, hipStream_t s,
                          const TimingHook& t);
hipError_t launch_merge(const MergeArgs& a, int head_dim, int part_dtype, int out_dtype,
                        hipStream_t s, const TimingHook& t);

}  // namespace sinkattn
