// Tile staging and block-to-work mapping shared by the forward and the
// backward kernels.
#pragma once

#include "device_common.h"
#include "sink_attn_internal.h"

namespace sinkattn {
namespace dev {

// Copy a [64 x D] bf16 tile of a THD tensor (row stride `stride` elements)
// straight from global memory into a swizzled LDS tile with gfx950's
// global_load_lds_dwordx4: no registers hold the data, so the next tile can
// be in flight during a whole step of MFMA work. Each such instruction
// writes 16 bytes per lane to consecutive LDS addresses (wave-uniform base
// + 16 * lane, checked on the hardware), i.e. one 1 KB run per wave. A lane
// therefore fetches the logical chunk that belongs at its physical position:
// chunk (lane % (D/8)) ^ swz(row). Every pass advances the row by a multiple
// of 16, which leaves swz(row) unchanged, so one offset per lane serves all
// passes. Rows at or past the end of the sequence fetch its last row (finite,
// in bounds; every consumer gives them zero weight). Completion is waited
// for with wait_vmem() before the barrier that publishes the tile.
template <int D, int THREADS = 256>
struct TileDma {
  static constexpr int kPer = 64 * D / 8 / THREADS;      // passes per tile
  static constexpr int kRowsPerPass = THREADS / (D / 8);
  static_assert(kRowsPerPass % 16 == 0, "a pass must keep the row swizzle");
  int lrow;             // this lane's row in pass 0
  int lcol;             // byte offset of the logical chunk this lane fetches
  int wave_off;         // byte offset of this wave's 1 KB run within a pass
  __device__ __forceinline__ void init() {
    lrow = threadIdx.x / (D / 8);
    lcol = (((threadIdx.x % (D / 8)) ^ swz<D>(lrow)) * 16);
    wave_off = __builtin_amdgcn_readfirstlane((threadIdx.x / 64) * 1024);
  }
  // rows [row0, row0 + 64) of the tensor at `base` into `tile`; the caller
  // guarantees row0 < nrows
  __device__ __forceinline__ void load(const bf16* base, int64_t stride, int row0, int nrows,
                                       char* tile) const {
    const char* p = reinterpret_cast<const char*>(base + (int64_t)row0 * stride);
    const int lim = nrows - row0 - 1;
    const int stride2 = (int)(stride * 2);
#pragma unroll
    for (int s = 0; s < kPer; ++s) {
      const int row = min(lrow + s * kRowsPerPass, lim);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(p + (uint32_t)(row * stride2 + lcol)),
          (__attribute__((address_space(3))) void*)(tile + s * THREADS * 16 + wave_off), 16, 0, 0);
    }
  }
};

// Head index for the j-th slot of the head-fastest block numbering. Blocks
// are spread over the 8 XCDs round robin (block id mod 8); with this map the
// q-heads of one kv group -- which read the same K/V -- share an XCD and
// its L2 whenever Hq is a multiple of 8.
__device__ __forceinline__ int head_of_slot(int j, int hq) {
  if ((hq & 7) == 0) return (j & 7) * (hq >> 3) + (j >> 3);
  return j;
}

}  // namespace dev
}  // namespace sinkattn
