// Tile staging and block-to-work mapping shared by the forward and the
// backward kernels.
#pragma once

#include "device_common.h"
#include "sink_attn_internal.h"

namespace sinkattn {
namespace dev {

// Stage a [64 x D] bf16 tile of rows [row0, row0 + 64) of a THD tensor
// (row stride `stride` elements) into registers; rows >= nrows read as 0.
template <int D>
struct TileLoader {
  static constexpr int kChunks = 64 * D / 8;           // 16-byte chunks per tile
  static constexpr int kPerThread = kChunks / 256;     // 4 (D=128) or 2 (D=64)
  u32x4 r[kPerThread];
  __device__ __forceinline__ void load(const bf16* base, int64_t stride, int row0,
                                       int nrows) {
#pragma unroll
    for (int s = 0; s < kPerThread; ++s) {
      const int u = threadIdx.x + 256 * s;
      const int row = u / (D / 8), c = u % (D / 8);
      if (row0 + row < nrows)
        r[s] = ld16(base + (int64_t)(row0 + row) * stride + c * 8);
      else
        r[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
#pragma unroll
    for (int s = 0; s < kPerThread; ++s) {
      const int u = threadIdx.x + 256 * s;
      lds_store_chunk<D>(tile, u / (D / 8), u % (D / 8), r[s]);
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
