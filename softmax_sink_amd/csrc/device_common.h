// Device-side building blocks for gfx950 (CDNA4): MFMA fragments, LDS tile
// swizzle, transposed LDS reads, wave-half exchange, exp2/log2.
//
// Lane layouts (checked on the hardware with an in-bounds probe):
//  * v_mfma_f32_32x32x16_bf16: lane l holds A[m = l%32][k = 8(l/32)+i] and
//    B[k = 8(l/32)+i][n = l%32], i = 0..7; the 16 results of lane l are
//    C[8(r/4) + 4(l/32) + r%4][l%32], r = 0..15.
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane 4a+c supplies the
//    address of 4 consecutive 16-bit elements (row a of a 4x16 block,
//    columns 4c..4c+3); lane n of the group receives column n of the 4 rows.
//  * v_permlane32_swap: returns (own, partner) for lanes 0..31 and
//    (partner, own) for lanes 32..63, where partner = lane ^ 32.
//
// Because every MFMA sums over its K slots, the order in which keys (or
// queries) are assigned to K slots is free as long as both operands agree.
// The kernels use the slot order that the 32x32 result layout produces:
// K slot i of lane half hl in chunk t is row 16t + 8(i/4) + 4hl + i%4. A
// probability tile computed as an MFMA result is then directly the B operand
// of the next MFMA, and the other operand is read with two transposed LDS
// reads (rows 16t + 4hl + e and 16t + 8 + 4hl + e).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace sinkattn {
namespace dev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Vectors of the 16-bit input types (bf16 or fp16): 8 elements are one
// MFMA operand fragment per lane, 4 elements one 8-byte store.
template <typename T> struct V16;
template <> struct V16<bf16> { typedef bf16x8 x8; typedef bf16x4 x4; };
template <> struct V16<f16> { typedef f16x8 x8; typedef f16x4 x4; };
template <typename T> using vec8 = typename V16<T>::x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_f16: the same lane layouts with fp16 operands.
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware v_exp_f32 (exact at -inf -> 0); e^x is obtained by
// the caller as 2^(x log2 e).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2 with the hardware v_log_f32 (x > 0).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane ^ 32.
__device__ __forceinline__ float half_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  const int lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// LDS tiles of 16-bit rows (D elements = D/8 16-byte chunks per row), stored
// without padding; the 16-byte chunk c of row r sits at chunk c ^ f(r).
// f makes both access patterns conflict-free over the 64 4-byte banks:
//   (a) 16 lanes reading the same chunk of 16 consecutive rows (ds_read_b128);
//   (b) a transposed read of 4 consecutive rows x 64 contiguous bytes.
// D = 128 (256-byte rows): f = 4(r%4) + (r/4)%4, a permutation of 0..15 on
//   any 16 consecutive rows whose upper two bits differ on 4 consecutive rows.
// D = 64 (128-byte rows, two rows per bank sweep): f = 4((r/2)%2) + (r/4)%4.
// D = 256: a tile is kept as two [rows x 128] slices (columns 0..127, then
//   128..255), each laid out as a D = 128 tile, so that every access pattern
//   and tile transfer of D = 128 carries over slice by slice.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "row swizzle of one slice");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
constexpr int kSliceCols = D > 128 ? 128 : D;                 // columns per slice
template <int D, int ROWS = 64>
constexpr int kSliceBytes = ROWS * kSliceCols<D> * 2;        // bytes per slice of ROWS rows

// Byte offset of the 16-byte chunk `chunk` (columns 8*chunk..+7) of row r
// of a tile of ROWS rows.
template <int D, int ROWS = 64>
__device__ __forceinline__ int chunk_off(int r, int chunk) {
  constexpr int DS = kSliceCols<D>;
  constexpr int CPS = DS / 8;                                 // chunks per slice row
  if constexpr (D > DS)
    return (chunk / CPS) * kSliceBytes<D, ROWS> + r * (DS * 2) + (((chunk % CPS) ^ swz<DS>(r)) << 4);
  else
    return r * (D * 2) + ((chunk ^ swz<D>(r)) << 4);
}

// Byte offset of element (r, col) (col a multiple of 4 elements).
template <int D, int ROWS = 64>
__device__ __forceinline__ int tile_off(int r, int col) {
  return chunk_off<D, ROWS>(r, col >> 3) + ((col & 7) << 1);
}

// 16-byte chunk (8 elements starting at column 8*chunk) of row r.
template <int D, typename T = bf16, int ROWS = 64>
__device__ __forceinline__ vec8<T> lds_row_chunk(const char* tile, int r, int chunk) {
  return *reinterpret_cast<const vec8<T>*>(tile + chunk_off<D, ROWS>(r, chunk));
}

template <int D>
__device__ __forceinline__ void lds_store_chunk(char* tile, int r, int chunk, u32x4 v) {
  *reinterpret_cast<u32x4*>(tile + chunk_off<D>(r, chunk)) = v;
}

__device__ __forceinline__ s16x4 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// MFMA operand whose K slots run down the rows of an LDS tile (rows
// row0 + 8(i/4) + 4hl + i%4, i = 0..7) and whose M/N index is column
// col0 + lane%32: two transposed reads.
template <int D, typename T = bf16, int ROWS = 64>
__device__ __forceinline__ vec8<T> lds_col_operand(const char* tile, int row0, int col0) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;          // 16-lane group
  const int hl = grp >> 1;            // lane half
  const int nu = lane & 15;
  const int r = row0 + 4 * hl + (nu >> 2);
  const int col = col0 + 16 * (grp & 1) + 4 * (nu & 3);
  s16x4 lo = ds_read_tr(tile + tile_off<D, ROWS>(r, col));
  s16x4 hi = ds_read_tr(tile + tile_off<D, ROWS>(r + 8, col));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(vec8<T>, v);
}

// Eight fp32 values -> 8 x T, round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32).
template <typename T = bf16>
__device__ __forceinline__ vec8<T> pack8(float a0, float a1, float a2, float a3,
                                         float a4, float a5, float a6, float a7) {
  vec8<T> r = {(T)a0, (T)a1, (T)a2, (T)a3, (T)a4, (T)a5, (T)a6, (T)a7};
  return r;
}

// Slots 8h..8h+7 of a 32x32 result fragment as the next MFMA's operand.
template <typename T = bf16>
__device__ __forceinline__ vec8<T> frag_half(const f32x16& c, int h) {
  return pack8<T>(c[8 * h + 0], c[8 * h + 1], c[8 * h + 2], c[8 * h + 3],
                  c[8 * h + 4], c[8 * h + 5], c[8 * h + 6], c[8 * h + 7]);
}

template <typename T = bf16>
__device__ __forceinline__ u32x2 pack4_bits(float a, float b, float c, float d) {
  typename V16<T>::x4 v = {(T)a, (T)b, (T)c, (T)d};
  return __builtin_bit_cast(u32x2, v);
}

// Wait for every outstanding vector-memory load (s_waitcnt vmcnt(0), other
// counters untouched). Placed before a tile loop whose entry can be reached
// with loads still in flight on some path, so that the compiler does not
// carry a conservative vmcnt(0) into every iteration, where it would also
// wait for the prefetch of the next tile.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Instruction-group directives for the machine scheduler
// (llvm.amdgcn.sched.group.barrier): the instructions of one scheduling
// region are placed in the order of the groups requested, e.g. "3 LDS
// reads, then 2 MFMAs and 1 LDS read, repeated", which keeps operand reads
// a few MFMAs ahead of their use instead of waiting on each one.
enum SchedMask : int {
  kSchedValu = 0x002,
  kSchedMfma = 0x008,
  kSchedDsRead = 0x100,
  kSchedDsWrite = 0x200,
};
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
// LEAD groups of READS LDS reads up front, then (MFMAS MFMAs, READS reads)
// until the reads run out, then the remaining MFMAs.
template <int NMFMA, int MFMAS, int READS, int LEAD>
__device__ __forceinline__ void sched_mfma_pipeline() {
  constexpr int kGroups = NMFMA / MFMAS;
  sched_group<kSchedDsRead, LEAD * READS>();
#pragma unroll
  for (int g = 0; g < kGroups - LEAD; ++g) {
    sched_group<kSchedMfma, MFMAS>();
    sched_group<kSchedDsRead, READS>();
  }
  sched_group<kSchedMfma, LEAD * MFMAS>();
}

// Wave priority around the MFMA-dense stretches of a tile step (s_setprio
// 1 before, 0 after): when the two waves of a SIMD both have an instruction
// ready, the one feeding the matrix pipe issues first, and the other's
// softmax / dS arithmetic fills the cycles the MFMAs leave free. Measured on
// the training step: 1-3% faster end to end (the forward, dK/dV and dQ
// kernels each a little faster), the prefill forward unchanged.
__device__ __forceinline__ void mfma_priority_high() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_priority_low() { __builtin_amdgcn_s_setprio(0); }

// Global 16-byte load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Kept key interval [jlo, jhi] of query row i (bottom-right aligned, clipped
// to [0, lk-1]); an empty interval has jhi < jlo.
__device__ __forceinline__ void row_key_range(int i, int lq, int lk, int causal,
                                              int wl, int wr, int& jlo, int& jhi) {
  const int pos = i + lk - lq;
  jlo = wl >= 0 ? max(0, pos - wl) : 0;
  int hi = lk - 1;
  if (causal) hi = min(hi, pos);
  else if (wr >= 0) hi = min(hi, pos + wr);
  jhi = hi;
  if (i >= lq) jhi = -1;
}

// Query rows [ilo, ihi] that keep key j (inverse of row_key_range).
__device__ __forceinline__ void key_row_range(int j, int lq, int lk, int causal,
                                              int wl, int wr, int& ilo, int& ihi) {
  const int off = lk - lq;
  int lo = 0, hi = lq - 1;
  if (causal) lo = max(lo, j - off);
  else if (wr >= 0) lo = max(lo, j - off - wr);
  if (wl >= 0) hi = min(hi, j - off + wl);
  if (j >= lk) hi = -1;
  ilo = lo;
  ihi = hi;
}

}  // namespace dev
}  // namespace sinkattn
