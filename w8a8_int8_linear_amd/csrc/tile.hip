// Copy of packed weight rows into the TILE16 layout read by the small-M
// kernel (gemv.hip): rows grouped in tiles of 16 and, within a tile, each
// 64-byte unit of K stored as 16 rows x 64 bytes = 1 KiB of consecutive
// memory, so that a transfer of one unit of a tile reads consecutive bytes.
// Pure data movement (offline, like packing); the scales are copied along.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launchers.h"

namespace convrot {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileThreads = 256;

// One thread per 16-byte chunk of the destination (a grid-stride loop):
// destination byte o is in tile o / (16 row_bytes), unit (o mod 16
// row_bytes) / 1024, row (o / 64) mod 16 of the tile, and byte
// 64 unit + o mod 64 of that row.
__global__ __launch_bounds__(kTileThreads) void tile_rows_kernel(const uint8_t* __restrict__ src, int64_t lds,
                                                                  uint8_t* __restrict__ dst, int64_t rows,
                                                                  int64_t row_bytes, const float* __restrict__ s_in,
                                                                  float* __restrict__ s_out) {
  const int64_t tile_bytes = 16 * row_bytes;
  const int64_t chunks = rows * row_bytes / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kTileThreads;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kTileThreads + threadIdx.x; c < chunks; c += stride) {
    const int64_t o = 16 * c;                 // destination byte
    const int64_t tile = o / tile_bytes;
    const int64_t w = o - tile * tile_bytes;  // byte within the tile
    const int64_t unit = w >> 10;             // 1 KiB per unit
    const int64_t r = (w >> 6) & 15;          // row within the tile
    const int64_t b = unit * 64 + (w & 63);   // byte within the row
    *reinterpret_cast<i32x4*>(dst + o) = *reinterpret_cast<const i32x4*>(src + (tile * 16 + r) * lds + b);
  }
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kTileThreads + threadIdx.x; i < rows; i += stride)
    s_out[i] = s_in[i];
}

}  // namespace

hipError_t launch_tile_rows(const uint8_t* src, int64_t lds, uint8_t* dst, int64_t rows, int64_t row_bytes,
                            const float* s_in, float* s_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t chunks = rows * row_bytes / 16;
  const int64_t blocks = std::min<int64_t>((chunks + kTileThreads - 1) / kTileThreads, 8192);
  hipLaunchKernelGGL(tile_rows_kernel, dim3(static_cast<unsigned>(std::max<int64_t>(blocks, 1))), dim3(kTileThreads),
                     0, stream, src, lds, dst, rows, row_bytes, s_in, s_out);
  return hipGetLastError();
}

}  // namespace convrot
