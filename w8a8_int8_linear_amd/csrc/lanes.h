// Lane exchanges, the unnormalised radix-4 butterfly and wavefront maxima
// shared by the pack kernel and the GEMM epilogue that computes the next
// layer's per-group maxima: both must evaluate the rotation with the same
// operations in the same order, so that their results agree bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {
namespace lanes {

// DPP control words.
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kQuadXor3 = 0x1B;  // quad_perm [3,2,1,0]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;  // lane ^ 8 within a row of 16
// ds_swizzle bit-mask mode: lane' = lane ^ xor_mask within 32 lanes.
constexpr int kSwzXor4 = 0x1F | (4 << 10);
constexpr int kSwzXor16 = 0x1F | (16 << 10);

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int PATTERN>
__device__ __forceinline__ float swz(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), PATTERN));
}
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Value held by lane ^ MASK (MASK a power of two below 64).
template <int MASK>
__device__ __forceinline__ float lane_xor(float x) {
  if constexpr (MASK == 1) return dpp<kQuadXor1>(x);
  else if constexpr (MASK == 2) return dpp<kQuadXor2>(x);
  else if constexpr (MASK == 4) return swz<kSwzXor4>(x);
  else if constexpr (MASK == 8) return dpp<kRowRor8>(x);
  else if constexpr (MASK == 16) return swz<kSwzXor16>(x);
  else return xor32(x);
}

// Unnormalised radix-4 butterfly (2 H4) on four registers.
__device__ __forceinline__ void bfly4(float& a0, float& a1, float& a2, float& a3) {
  const float s = (a0 + a1) + (a2 + a3);
  const float b0 = fmaf(-2.f, a3, s);
  const float b1 = fmaf(-2.f, a2, s);
  const float b2 = fmaf(-2.f, a1, s);
  const float b3 = fmaf(-2.f, a0, s);
  a0 = b0; a1 = b1; a2 = b2; a3 = b3;
}

// Maximum over the wavefront of non-negative values.  For those the IEEE
// bit patterns order like unsigned integers, so the reduction runs on the
// bits (an unsigned max takes its lane exchange as a DPP operand and needs
// none of the NaN canonicalisation a float max would add at every step).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t m) {
  m = max(m, dpp_u<kQuadXor1>(m));
  m = max(m, dpp_u<kQuadXor2>(m));
  m = max(m, dpp_u<kRowRor4>(m));
  m = max(m, dpp_u<kRowRor8>(m));
  m = max(m, static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(m), kSwzXor16)));
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32)));
  return m;
}

}  // namespace lanes
}  // namespace convrot
