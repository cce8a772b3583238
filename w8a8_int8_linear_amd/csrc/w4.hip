// int4 weight codes (nibble pairs) expanded to int8 codes, for gfx950.
//
// The format is the int4 ConvRot weight of the stable-diffusion.cpp PR "load
// ConvRot int4 and per-channel int8 safetensors" (sections "Solution" and
// "The rotation"): codes in [-7, 7], two per byte, element 2j in the low and
// 2j + 1 in the high nibble of byte j, each as 4-bit two's complement.  The
// tiled matrix-core kernel takes int8 codes, so a linear with more than a
// handful of rows expands the weight once per call into a workspace; the
// bytes moved (K / 2 read and K written per row) are small against that
// GEMM's work.  HBM bound: each thread turns one 8-byte load into one
// 16-byte store, consecutive threads on consecutive bytes of a row.
#include <hip/hip_runtime.h>

#include "launchers.h"
#include "w4_codec.h"

namespace convrot {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// units = K / 16 8-byte units per row; total = rows * units threads of work.
__global__ __launch_bounds__(256) void unpack_w4_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                        int8_t* __restrict__ dst, int64_t ldd, int64_t units,
                                                        int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / units, unit = i % units;
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q + row * ldq + 8 * unit));
  *reinterpret_cast<w4_i32x4*>(dst + row * ldd + 16 * unit) = expand_w4(w.x, w.y);
}

}  // namespace

hipError_t launch_unpack_w4(const uint8_t* q, int64_t ldq, int64_t rows, int64_t K, int8_t* dst, int64_t ldd,
                            hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t units = K / 16;
  const int64_t total = rows * units;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(unpack_w4_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, q, ldq, dst, ldd,
                     units, total);
  return hipGetLastError();
}

}  // namespace convrot
