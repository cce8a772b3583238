// Epilogue pieces shared by the tiled and the small-M linear kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Per-launch epilogue operands.  int8 mode: Y = A sa[m] sb[n] + bias[n];
// gated: the up weight (B2, its scales sb2 and bias bias2) shares the packed
// activation.
struct EpiArgs {
  const float* sa;
  const float* sb;
  const float* bias;
  const uint8_t* B2;
  int64_t ldb2;
  const float* sb2;
  const float* bias2;
};

// Activations of the fused epilogue: 0 none, 1 GELU (erf form), 2 GELU
// (tanh form); the erf and tanh are the device math library's.
template <int ACT>
__device__ __forceinline__ float activation(float y) {
  if constexpr (ACT == 1) {
    return 0.5f * y * (1.f + erff(y * 0.70710678118654752f));
  } else if constexpr (ACT == 2) {
    const float u = 0.79788456080286536f * fmaf(0.044715f * y, y * y, y);
    return 0.5f * y * (1.f + tanhf(u));
  } else {
    return y;
  }
}


}  // namespace convrot
