// Data-free smoothing of an FFN's intermediate channels, offline, gfx950.
//
// "Add experimental W8A8 MatMul with optional QuaRot-style rotation"
// (gemma.cpp issue), maintainer's review comment: before the rotation, scale
// the weights without calibration data -- by max norms, or by the square
// root of the ratio of the W_up to W_down L2 column norms -- so that the
// quantisation range shrinks; the factor is pulled into the per-row scales.
// For intermediate channel j (row j of W_up [F, K], column j of W_down
// [K_out, F]):
//   s_j = sqrt(n_up[j] / n_down[j])   (n = L2 norm or largest magnitude;
//                                      1 where either is 0)
//   W_up'[j, :] = W_up[j, :] / s_j,   W_down'[:, j] = W_down[:, j] * s_j
// which gives both the norm sqrt(n_up n_down) and leaves a gated FFN
// (h = act(gate) * up) unchanged.  The scaled weights are then packed as
// usual; at run time nothing changes.
//
// Offline and small next to a pack, so the kernels favour exactness over
// speed: norms accumulate in fp64 (one workgroup per channel, the W_down
// column read with a stride), s is rounded once to fp32, and each scaled
// weight is the fp64 quotient or product with that s, rounded once to fp32.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launchers.h"

namespace convrot {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ double load_elt(const T* p, int64_t i);
template <>
__device__ __forceinline__ double load_elt<float>(const float* p, int64_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double load_elt<uint16_t>(const uint16_t* p, int64_t i) {
  return static_cast<double>(__builtin_bit_cast(float, static_cast<uint32_t>(p[i]) << 16));
}

// Sum (L2: of squares) or max (of magnitudes) over the workgroup.
template <bool MAX>
__device__ double block_reduce(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const double w = __shfl_xor(v, o);
    v = MAX ? fmax(v, w) : v + w;
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = MAX ? fmax(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

template <typename TU, typename TD, bool MAX>
__global__ __launch_bounds__(kThreads) void smooth_scales_kernel(const TU* __restrict__ up, int64_t ldu,
                                                                 const TD* __restrict__ dn, int64_t ldd, int64_t K,
                                                                 int64_t K_out, float* __restrict__ s) {
  __shared__ double red[kThreads / 64];
  const int64_t j = blockIdx.x;
  double a = 0.0, b = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    const double v = load_elt<TU>(up, j * ldu + k);
    a = MAX ? fmax(a, fabs(v)) : a + v * v;
  }
  for (int64_t i = threadIdx.x; i < K_out; i += kThreads) {
    const double v = load_elt<TD>(dn, i * ldd + j);
    b = MAX ? fmax(b, fabs(v)) : b + v * v;
  }
  a = block_reduce<MAX>(a, red);
  b = block_reduce<MAX>(b, red);
  if (threadIdx.x == 0) {
    const double n_up = MAX ? a : sqrt(a), n_dn = MAX ? b : sqrt(b);
    s[j] = (n_up > 0.0 && n_dn > 0.0) ? static_cast<float>(sqrt(n_up / n_dn)) : 1.0f;
  }
}

// out[r, c] = in[r, c] / s[r] (DIV_ROWS) or in[r, c] * s[c], fp64, rounded once.
template <typename T, bool DIV_ROWS>
__global__ __launch_bounds__(kThreads) void smooth_apply_kernel(const T* __restrict__ in, int64_t ldi, int64_t rows,
                                                                int64_t cols, const float* __restrict__ s,
                                                                float* __restrict__ out, int64_t ldo) {
  const int64_t n = rows * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t r = i / cols, c = i % cols;
    const double v = load_elt<T>(in, r * ldi + c);
    out[r * ldo + c] = static_cast<float>(DIV_ROWS ? v / static_cast<double>(s[r]) : v * static_cast<double>(s[c]));
  }
}

template <typename TU, typename TD>
hipError_t scales_typed(bool max_norm, const void* up, int64_t ldu, const void* dn, int64_t ldd, int64_t F, int64_t K,
                        int64_t K_out, float* s, hipStream_t stream) {
  const auto* u = static_cast<const TU*>(up);
  const auto* d = static_cast<const TD*>(dn);
  if (max_norm)
    hipLaunchKernelGGL((smooth_scales_kernel<TU, TD, true>), dim3(static_cast<unsigned>(F)), dim3(kThreads), 0,
                       stream, u, ldu, d, ldd, K, K_out, s);
  else
    hipLaunchKernelGGL((smooth_scales_kernel<TU, TD, false>), dim3(static_cast<unsigned>(F)), dim3(kThreads), 0,
                       stream, u, ldu, d, ldd, K, K_out, s);
  return hipGetLastError();
}

template <typename T, bool DIV_ROWS>
hipError_t apply_typed(const void* in, int64_t ldi, int64_t rows, int64_t cols, const float* s, float* out,
                       int64_t ldo, hipStream_t stream) {
  const int64_t n = rows * cols;
  const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 65536);
  hipLaunchKernelGGL((smooth_apply_kernel<T, DIV_ROWS>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(in), ldi, rows, cols, s, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_smooth_ffn(const void* up, Elt up_dt, int64_t ldu, const void* dn, Elt dn_dt, int64_t ldd, int64_t F,
                             int64_t K, int64_t K_out, bool max_norm, float* s, float* up_out, int64_t ldu_out,
                             float* dn_out, int64_t ldd_out, hipStream_t stream) {
  if (F == 0) return hipSuccess;
  const bool ub = up_dt == Elt::BF16, db = dn_dt == Elt::BF16;
  hipError_t e = ub ? (db ? scales_typed<uint16_t, uint16_t>(max_norm, up, ldu, dn, ldd, F, K, K_out, s, stream)
                          : scales_typed<uint16_t, float>(max_norm, up, ldu, dn, ldd, F, K, K_out, s, stream))
                    : (db ? scales_typed<float, uint16_t>(max_norm, up, ldu, dn, ldd, F, K, K_out, s, stream)
                          : scales_typed<float, float>(max_norm, up, ldu, dn, ldd, F, K, K_out, s, stream));
  if (e != hipSuccess) return e;
  if (up_out != nullptr) {
    e = ub ? apply_typed<uint16_t, true>(up, ldu, F, K, s, up_out, ldu_out, stream)
           : apply_typed<float, true>(up, ldu, F, K, s, up_out, ldu_out, stream);
    if (e != hipSuccess) return e;
  }
  if (dn_out != nullptr) {
    e = db ? apply_typed<uint16_t, false>(dn, ldd, K_out, F, s, dn_out, ldd_out, stream)
           : apply_typed<float, false>(dn, ldd, K_out, F, s, dn_out, ldd_out, stream);
  }
  return e;
}

}  // namespace convrot
