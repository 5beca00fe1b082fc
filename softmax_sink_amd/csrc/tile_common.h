// Tile staging and block-to-work mapping shared by the forward and the
// backward kernels.
#pragma once

#include "device_common.h"
#include "sink_attn_internal.h"

namespace sinkattn {
namespace dev {

// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data
// format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// Copy a [64 x D] tile of 16-bit elements of a THD tensor (row stride `stride` elements)
// straight from global memory into a swizzled LDS tile with gfx950's
// buffer_load_dwordx4 ... lds: no registers hold the data, so the next tile
// can be in flight during a whole step of MFMA work. Each such instruction
// writes 16 bytes per lane to consecutive LDS addresses (wave-uniform base
// in M0 + 16 * lane, checked on the hardware), i.e. one 1 KB run per wave.
//
// The instruction is issued from inline assembly, invisible to the
// compiler's wait-count tracking. Through the builtin, the compiler cannot
// tell the tile in flight from the tiles being read (the transposed LDS
// reads carry no alias information), so it waits for the whole prefetch
// (vmcnt(0)) before the first such read of every step, and a FLAT-encoded
// form additionally turns every LDS wait into lgkmcnt(0). The kernels
// instead wait for their prefetches explicitly (wait_vmem() before the
// barrier that publishes a tile) and never touch a tile in flight. The
// assembly has no outputs; its address operands are read at issue, the LDS
// destination comes in M0 as an input operand (the compiler writes M0
// itself, so it knows the register's value), and it clobbers memory. A lane
// therefore fetches the logical chunk that belongs at its physical position:
// chunk (lane % (D/8)) ^ swz(row). Every pass advances the row by a multiple
// of 16, which leaves swz(row) unchanged, so one offset per lane serves all
// passes. Rows at or past the end of the sequence fetch its last row (finite,
// in bounds; every consumer gives them zero weight). Completion is waited
// for with wait_vmem() before the barrier that publishes the tile.
// A D = 256 tile moves as its two 128-column slices, one after the other.
template <int D, int THREADS = 256, int ROWS = 64>
struct TileDma {
  static constexpr int DS = kSliceCols<D>;
  static constexpr int kSlices = D / DS;
  static constexpr int kPer = ROWS * DS / 8 / THREADS;   // passes per slice
  static_assert(kPer >= 1 && ROWS * DS / 8 % THREADS == 0, "whole passes");
  static constexpr int kRowsPerPass = THREADS / (DS / 8);
  static_assert(kRowsPerPass % 16 == 0, "a pass must keep the row swizzle");
  int lrow;             // this lane's row in pass 0
  int lcol;             // byte offset of the logical chunk this lane fetches
  int wave_off;         // byte offset of this wave's 1 KB run within a pass
  __device__ __forceinline__ void init() {
    lrow = threadIdx.x / (DS / 8);
    lcol = (((threadIdx.x % (DS / 8)) ^ swz<DS>(lrow)) * 16);
    wave_off = __builtin_amdgcn_readfirstlane((threadIdx.x / 64) * 1024);
  }
  // One tile transfer, prepared (uniform values only) and then issued in
  // parts, so that a kernel can spread the issue over its MFMA work: the
  // issue of a wave stalls while the memory pipeline is backed up.
  struct Tile {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lds;       // LDS address of this wave's run in pass 0
    int lim;            // last valid row, relative to the tile's first row
    int stride2;        // row stride in bytes
  };
  // rows [row0, row0 + 64) of one slice (columns from `base` on) of the
  // tensor at `base` into `tile`; the caller guarantees row0 < nrows
  template <typename T>
  __device__ __forceinline__ Tile prepare(const T* base, int64_t stride, int row0, int nrows,
                                          char* tile) const {
    Tile t;
    // raw buffer over the tile's first row; rows are clamped to lim, so the
    // range check (2 GiB) never trims a load
    t.rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(base + (int64_t)row0 * stride), (short)0, 0x7FFFFFFF, kBufferWord3);
    t.lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(tile + wave_off));
    t.lim = nrows - row0 - 1;
    t.stride2 = (int)(stride * 2);
    return t;
  }
  // passes [S0, S1) of a prepared tile
  template <int S0, int S1>
  __device__ __forceinline__ void issue(const Tile& t) const {
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      const int row = min(lrow + s * kRowsPerPass, t.lim);
      const uint32_t voff = (uint32_t)(row * t.stride2 + lcol);
      asm volatile(
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %1, %0, 0 offen lds"
          :
          : "s"(t.rsrc), "v"(voff), "{m0}"(t.lds + s * THREADS * 16)
          : "memory");
    }
  }
  template <typename T>
  __device__ __forceinline__ void load(const T* base, int64_t stride, int row0, int nrows,
                                       char* tile) const {
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl)
      issue<0, kPer>(prepare(base + sl * DS, stride, row0, nrows, tile + sl * (ROWS * DS * 2)));
  }
};

// The same [64 x D] tile transfer for keys or values that live in a paged
// cache: row r of the sequence is slot (r - k_lo + off0) % block_size of the
// page pages[(r - k_lo + off0) / block_size], where `pages` is an LDS copy of
// the block-table entries of the work item, starting with the page that
// holds its first key k_lo at slot off0; (page p, slot s) of the kv-head
// sits at element p * page_stride + s * row_stride + head_off of the cache. Rows past `row_last` fetch row_last. Each lane computes its own
// 64-bit row address, so the FLAT form global_load_lds_dwordx4 is used, again
// from inline assembly (no outputs; M0 an input operand; clobbers memory). The division by
// block_size is a multiply-high with magic = ceil(2^32 / block_size), exact
// here because the numerator stays below 2^12.
template <int D, int THREADS = 256>
struct PagedTileDma {
  static constexpr int DS = kSliceCols<D>;
  static constexpr int kSlices = D / DS;
  static constexpr int kPer = 64 * DS / 8 / THREADS;
  static constexpr int kRowsPerPass = THREADS / (DS / 8);
  static_assert(kRowsPerPass % 16 == 0, "a pass must keep the row swizzle");
  int lrow, lcol, wave_off;
  __device__ __forceinline__ void init() {
    lrow = threadIdx.x / (DS / 8);
    lcol = (((threadIdx.x % (DS / 8)) ^ swz<DS>(lrow)) * 16);
    wave_off = __builtin_amdgcn_readfirstlane((threadIdx.x / 64) * 1024);
  }
  // The K and V tiles of the same rows: each lane finds its row's page slot
  // once and issues both transfers (the two caches share their layout).
  template <typename T>
  __device__ __forceinline__ void load_kv(const T* kcache, const T* vcache, int64_t head_off,
                                          int64_t row_stride, int64_t page_stride, const int* pages,
                                          int off0, int k_lo, int row0, int row_last, int block_size,
                                          uint32_t magic, char* ktile, char* vtile) const {
    const uint32_t kl0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ktile + wave_off));
    const uint32_t vl0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(vtile + wave_off));
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int row = min(row0 + lrow + s * kRowsPerPass, row_last);
      const uint32_t num = (uint32_t)(row - k_lo + off0);
      const uint32_t pi = __umulhi(num, magic);
      const int slot = (int)(num - pi * (uint32_t)block_size);
      const int64_t elem = (int64_t)pages[pi] * page_stride + slot * row_stride + head_off;
      const char* ks = reinterpret_cast<const char*>(kcache + elem) + lcol;
      const char* vs = reinterpret_cast<const char*>(vcache + elem) + lcol;
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) {
        asm volatile(
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off"
            :
            : "v"(ks + sl * DS * 2), "{m0}"(kl0 + sl * kSliceBytes<D> + s * THREADS * 16)
            : "memory");
        asm volatile(
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off"
            :
            : "v"(vs + sl * DS * 2), "{m0}"(vl0 + sl * kSliceBytes<D> + s * THREADS * 16)
            : "memory");
      }
    }
  }
};

// Rows of sequence b (see Geometry): first row and row count, for the query
// side and the key side.
template <class A>
__device__ __forceinline__ int q_start(const A& a, int b) {
  return a.g.seq_q ? b * a.g.seq_q : a.cu_q[b];
}
template <class A>
__device__ __forceinline__ int q_len(const A& a, int b) {
  return a.g.seq_q ? (a.g.used_q ? a.g.used_q[b] : a.g.seq_q) : a.cu_q[b + 1] - a.cu_q[b];
}
template <class A>
__device__ __forceinline__ int k_start(const A& a, int b) {
  return a.g.seq_k ? b * a.g.seq_k : a.cu_k[b];
}
template <class A>
__device__ __forceinline__ int k_len(const A& a, int b) {
  return a.g.seq_k ? (a.g.used_k ? a.g.used_k[b] : a.g.seq_k) : a.cu_k[b + 1] - a.cu_k[b];
}
// Sequence and in-sequence row of query row t of the tensors (rows past a
// sequence's length in a padded layout give i >= q_len).
template <class A>
__device__ __forceinline__ void q_row_of(const A& a, int t, int& b, int& i) {
  if (a.g.seq_q) {
    b = t / a.g.seq_q;
    i = t - b * a.g.seq_q;
    return;
  }
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_q[mid] <= t) lo = mid; else hi = mid;
  }
  b = lo;
  i = t - a.cu_q[b];
}

// The same for key row t.
template <class A>
__device__ __forceinline__ void k_row_of(const A& a, int t, int& b, int& j) {
  if (a.g.seq_k) {
    b = t / a.g.seq_k;
    j = t - b * a.g.seq_k;
    return;
  }
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_k[mid] <= t) lo = mid; else hi = mid;
  }
  b = lo;
  j = t - a.cu_k[b];
}

// Head index for the j-th slot of the head-fastest block numbering. Blocks
// are spread over the 8 XCDs round robin (block id mod 8); with this map the
// q-heads of one kv group -- which read the same K/V -- share an XCD and
// its L2 whenever Hq is a multiple of 8.
__device__ __forceinline__ int head_of_slot(int j, int hq) {
  if ((hq & 7) == 0) return (j & 7) * (hq >> 3) + (j >> 3);
  return j;
}

// Store a [128 x D] result tile held in the MFMA output layout of four
// waves -- row r = 32w + c of the tile in lane (hl, c) of wave w (thread
// `tid` = 64w + 32hl + c of the group), column 32n + 8g + 4hl + e in
// acc[n][4g + e] -- scaled and rounded to T, into rows [0, nrows) of `dst`
// (row stride `stride` elements), through 128 * D * 2 bytes of LDS that the
// caller guarantees idle (no transfer in flight, no wave still reading).
// First each lane puts its 8-byte pieces into 16-byte granules of its row
// (granule j of row r at j ^ (r & SW), so that the 32 rows of a wave spread
// over the banks); after a barrier, D/8 threads store each row, 16 bytes
// apiece, so that every store instruction writes whole rows. Written
// straight from the MFMA layout instead, every store instruction of a wave
// covered 16 bytes of 32 different rows, and issuing a tile's stores took
// about 4000 cycles.
template <int D> struct TileRows {
  static constexpr int GR = D / 8;             // 16-byte granules per row
  static constexpr int SW = (GR < 16 ? GR : 16) - 1;
  static constexpr int RPP = 256 / GR;         // rows per store pass
  static constexpr int kBytes = 128 * D * 2;
};
template <int D, typename T>
__device__ __forceinline__ void tile_rows_to_lds(const f32x16* acc, float scale, char* lds, int tid) {
  using R = TileRows<D>;
  const int hl = (tid >> 5) & 1, r = (tid >> 6) * 32 + (tid & 31);
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = 4 * n + g;                 // granule of column 32n + 8g + 4hl
      *reinterpret_cast<u32x2*>(lds + r * (D * 2) + ((j ^ (r & R::SW)) * 16) + hl * 8) =
          pack4_bits<T>(acc[n][4 * g] * scale, acc[n][4 * g + 1] * scale,
                        acc[n][4 * g + 2] * scale, acc[n][4 * g + 3] * scale);
    }
}
template <int D, typename T>
__device__ __forceinline__ void tile_rows_from_lds(const char* lds, T* dst, int64_t stride, int nrows,
                                                   int tid) {
  using R = TileRows<D>;
  const int tr = tid / R::GR, tg = tid % R::GR;
#pragma unroll
  for (int r0 = 0; r0 < 128; r0 += R::RPP) {
    const int rr = r0 + tr;
    if (rr < nrows)
      *reinterpret_cast<u32x4*>(dst + (int64_t)rr * stride + tg * 8) =
          *reinterpret_cast<const u32x4*>(lds + rr * (D * 2) + ((tg ^ (rr & R::SW)) * 16));
  }
}
// Both halves for a 256-thread block.
template <int D, typename T>
__device__ __forceinline__ void store_tile_rows(const f32x16* acc, float scale, char* lds, T* dst,
                                                int64_t stride, int nrows) {
  tile_rows_to_lds<D, T>(acc, scale, lds, threadIdx.x);
  __syncthreads();
  tile_rows_from_lds<D, T>(lds, dst, stride, nrows, threadIdx.x);
}

// Work item and kv-head of split-KV block `id` (grid n_items x nh). The nh
// kv-heads of one key chunk read disjoint 2*D-byte pieces of the same K and
// V rows; they go to the same XCD (block id mod 8), one after the other, so
// that the whole rows are fetched close together in time. Items come in
// groups of 8, one item of each group per XCD; items past the last whole
// group take the plain order. Measured on the decode stream (8 kv-heads,
// 256-byte pieces of 2 KB rows): 6.05 TB/s against 5.70 TB/s for a grid
// with the heads of a chunk on 8 different XCDs.
__device__ __forceinline__ void chunk_work(int id, int n_items, int nh, int& item, int& h) {
  const int full = (n_items >> 3) * 8 * nh;      // blocks of the whole groups
  if (id < full) {
    const int x = id & 7, u = id >> 3;
    h = u % nh;
    item = (u / nh) * 8 + x;
    return;
  }
  item = id / nh;
  h = id % nh;
}

}  // namespace dev
}  // namespace sinkattn
