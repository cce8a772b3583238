// Small-M (decode) quantised linear for gfx950: the same result as the tiled
// GEMM (exact int32 A = Qx Qw^T, then Y = A s_x[r] s_w[o] + b[o]; "INT8
// Convrot Safetensors", "Runtime activation quantization"), organised to
// stream the int8 weight once at full bandwidth.
//
// With M <= 16 the work is bound by reading Qw (N*K bytes), so the kernel
// is built around the weight stream rather than around reuse:
//  * one workgroup per 16 output features; its 4 waves split K between
//    them (wave w takes 64-byte steps w, w+4, ...);
//  * every step is one v_mfma_i32_16x16x64_i8 whose row operand is 16 weight
//    rows (16 bytes per lane, loaded straight from global memory into
//    VGPRs, no LDS) and whose column operand is the (at most 16) activation
//    rows; lanes for activation rows >= M re-read the last row and their
//    outputs are dropped;
//  * steps are unrolled by 4 so each lane keeps 64 bytes of weight loads in
//    flight;
//  * the 4 partial accumulators are summed exactly through LDS and wave 0
//    applies the epilogue.
#include <hip/hip_runtime.h>

#include "launchers.h"

namespace convrot {
namespace {

// Four consecutive outputs go out as one vector store when aligned for it.
template <typename T>
__device__ __forceinline__ bool vec_ok(const T* p) {
  return (reinterpret_cast<uintptr_t>(p) & (4 * sizeof(T) - 1)) == 0;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = 4;

template <int OUT, bool KTAIL>
__global__ __launch_bounds__(kThreads) void gemv_i8_kernel(
    const int8_t* __restrict__ A, int64_t lda, const int8_t* __restrict__ B, int64_t ldb,
    const float* __restrict__ sa, const float* __restrict__ sb, const float* __restrict__ bias, int M, int N,
    int K, void* __restrict__ C, int64_t ldc) {
  __shared__ i32x4 partial[kWaves - 1][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int row = lane & 15;
  const int ch = lane >> 4;

  const int8_t* wrow = B + static_cast<int64_t>(min(n0 + row, N - 1)) * ldb + ch * 16;
  const int8_t* xrow = A + static_cast<int64_t>(min(row, M - 1)) * lda + ch * 16;

  i32x4 acc = {0, 0, 0, 0};
  const int nsteps = (K + 63) / 64;
  int s = wid;
  for (; s + kWaves * (kUnroll - 1) < nsteps; s += kWaves * kUnroll) {
    i32x4 w[kUnroll], x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = (s + kWaves * u) * 64;
      if (KTAIL && k + ch * 16 >= K) {
        w[u] = i32x4{0, 0, 0, 0};
        x[u] = i32x4{0, 0, 0, 0};
      } else {
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow + k));
        x[u] = *reinterpret_cast<const i32x4*>(xrow + k);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], x[u], acc, 0, 0, 0);
  }
  for (; s < nsteps; s += kWaves) {
    const int k = s * 64;
    i32x4 w = {0, 0, 0, 0}, x = {0, 0, 0, 0};
    if (!KTAIL || k + ch * 16 < K) {
      w = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow + k));
      x = *reinterpret_cast<const i32x4*>(xrow + k);
    }
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, acc, 0, 0, 0);
  }

  if (wid > 0) partial[wid - 1][lane] = acc;
  __syncthreads();
  if (wid != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) acc += partial[w][lane];

  // Lane holds output row m = lane & 15 and features n0 + 4 (lane >> 4) + r.
  const int m = row;
  const int n = n0 + 4 * ch;
  if (m >= M || n >= N) return;
  if constexpr (OUT == 2) {
    int32_t* out = static_cast<int32_t*>(C) + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N && vec_ok(out)) {
      *reinterpret_cast<i32x4*>(out) = acc;
    } else {
      for (int r = 0; r < 4 && n + r < N; ++r) out[r] = acc[r];
    }
    return;
  } else {
    const float s_row = sa[m];
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      y[r] = fmaf(static_cast<float>(acc[r]), s_row * sb[nn], bias ? bias[nn] : 0.f);
    }
    if constexpr (OUT == 0) {
      float* out = static_cast<float*>(C) + static_cast<int64_t>(m) * ldc + n;
      if (n + 3 < N && vec_ok(out)) {
        *reinterpret_cast<f32x4*>(out) = f32x4{y[0], y[1], y[2], y[3]};
      } else {
        for (int r = 0; r < 4 && n + r < N; ++r) out[r] = y[r];
      }
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      __bf16* out = static_cast<__bf16*>(C) + static_cast<int64_t>(m) * ldc + n;
      if (n + 3 < N && vec_ok(out)) {
        *reinterpret_cast<bf16x4*>(out) = bf16x4{static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1]),
                                                 static_cast<__bf16>(y[2]), static_cast<__bf16>(y[3])};
      } else {
        for (int r = 0; r < 4 && n + r < N; ++r) out[r] = static_cast<__bf16>(y[r]);
      }
    }
  }
}

template <int OUT>
hipError_t launch_out(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa, const float* sb,
                      const float* bias, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                      hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + 15) / 16));
  if (K % 64 == 0) {
    hipLaunchKernelGGL((gemv_i8_kernel<OUT, false>), grid, dim3(kThreads), 0, stream, A, lda, B, ldb, sa, sb, bias,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), C, ldc);
  } else {
    hipLaunchKernelGGL((gemv_i8_kernel<OUT, true>), grid, dim3(kThreads), 0, stream, A, lda, B, ldb, sa, sb, bias,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), C, ldc);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, int64_t M, int64_t N, int64_t K, void* C, Elt out,
                          int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  switch (out) {
    case Elt::F32: return launch_out<0>(A, lda, B, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
    case Elt::BF16: return launch_out<1>(A, lda, B, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
    default: return launch_out<2>(A, lda, B, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
  }
}

}  // namespace convrot
