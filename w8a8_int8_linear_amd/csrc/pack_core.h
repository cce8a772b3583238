// Per-chunk steps of the pack (group rotation, row maximum, int8 codes),
// shared by the pack kernel (pack_rows.hip) and the small-M linear that
// packs its own activation rows (gemv.hip), so that both give every code
// and scale with the same operations in the same order.
//
// A chunk is 16 contiguous features held by one lane.  A G-group spans
// G / 16 consecutive lanes of one wavefront (G >= 16), whose chunks follow
// chunk_in_group: the regular kind keeps base-4 digit 0 of the lane's
// position as is and Gray-codes digits 1 and 2, so that the partner holding
// digit 3 - d of a lane exchange is always lane ^ 3, ^ 8 or ^ 32; the
// randomized kind keeps the identity order for its radix-2 exchanges.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lanes.h"

namespace convrot {
namespace pack {

using namespace lanes;

constexpr int kChunk = 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Radix-4 butterfly whose digit lives in lane bits (2k, 2k+1).
// k = 0: identity digit order within a quad, partner at lane ^ 3.
// k = 1: Gray-coded digit in lane bits 2-3, partner at lane ^ 8.
// k = 2: Gray-coded digit in lane bits 4-5, partner at lane ^ 32.
// With the digit d of this lane and 3 - d held by the partner, the output
// s - 2 a_{3-d} equals (a_d - a_{3-d}) + (sum of the other pair), and the
// other pair's sum is held by the lanes one exchange away (lane ^ 1 in a
// quad, a rotation by 4 within 16 lanes for the Gray-coded digit 1, lane ^ 16
// for digit 2).  That is three two-operand instructions per element, each
// taking its lane exchange as a DPP source operand.
template <int K>
__device__ __forceinline__ float bfly4_lanes(float x) {
  if constexpr (K == 0) {
    const float u = x + dpp<kQuadXor3>(x);
    const float w = x - dpp<kQuadXor3>(x);
    return w + dpp<kQuadXor1>(u);
  } else if constexpr (K == 1) {
    const float u = x + dpp<kRowRor8>(x);
    const float w = x - dpp<kRowRor8>(x);
    return w + dpp<kRowRor4>(u);
  } else {
    const float p = xor32(x);
    const float u = x + p;
    const float w = x - p;
    return w + swz<kSwzXor16>(u);
  }
}

// Radix-2 (Sylvester) butterfly across lane bit b: the lane with the bit
// clear keeps a + c, the other keeps a - c (a = low lane's value).
template <int MASK>
__device__ __forceinline__ float bfly2_lanes(float x, int lane) {
  const float p = lane_xor<MASK>(x);
  return (lane & MASK) ? (p - x) : (x + p);
}

__device__ __forceinline__ int gray2(int m) { return m ^ (m >> 1); }

// Position of a lane's chunk inside its group.
template <bool RAND>
__device__ __forceinline__ int chunk_in_group(int pos) {
  if constexpr (RAND) {
    return pos;
  } else {
    return (pos & 3) + 4 * gray2((pos >> 2) & 3) + 16 * gray2((pos >> 4) & 3);
  }
}

// Rows are accessed through buffer resources whose size is the row's valid
// bytes: a load past the end returns zeros and a store past the end is
// dropped, so chunks beyond K (threads rounded up to whole wavefronts) need
// no test, no zero fill and no store guard.  Word 3 is the raw-buffer
// default (32-bit data format).  Cache policy: non-temporal, the row is
// touched once.
constexpr int kBufWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufWord3);
}

template <typename InT>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t r, int elem_off, float v[kChunk]);

// The 16 bf16 features of a chunk, as two 16-byte words, widened to fp32
// (exact: a bf16 value is the high half of its fp32 value).
__device__ __forceinline__ void bf16_words_to_chunk(u32x4 a, u32x4 b, float v[kChunk]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = as_f(w[i] << 16);
    v[2 * i + 1] = as_f(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load_chunk<uint16_t>(__amdgpu_buffer_rsrc_t r, int elem_off, float v[kChunk]) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * elem_off, 0, kNonTemporal);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * elem_off + 16, 0, kNonTemporal);
  bf16_words_to_chunk(a, b, v);
}

template <>
__device__ __forceinline__ void load_chunk<float>(__amdgpu_buffer_rsrc_t r, int elem_off, float v[kChunk]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, 4 * elem_off + 16 * i, 0, kNonTemporal);
    v[4 * i] = as_f(a.x); v[4 * i + 1] = as_f(a.y); v[4 * i + 2] = as_f(a.z); v[4 * i + 3] = as_f(a.w);
  }
}

// Randomized kind, first step: the chunk's +-1 signs (K bytes of int8 at
// `sr`, 16 of them per chunk) applied to its 16 features.
__device__ __forceinline__ u32x4 load_signs(__amdgpu_buffer_rsrc_t sr, int elem_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(sr, elem_off, 0, 0);
}

__device__ __forceinline__ void apply_sign_words(u32x4 sv, float v[kChunk]) {
  const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
  for (int e = 0; e < kChunk; ++e) {
    const int8_t sgn = static_cast<int8_t>((w[e >> 2] >> (8 * (e & 3))) & 0xFF);
    v[e] = sgn < 0 ? -v[e] : v[e];
  }
}

__device__ __forceinline__ void apply_signs(__amdgpu_buffer_rsrc_t sr, int elem_off, float v[kChunk]) {
  apply_sign_words(load_signs(sr, elem_off), v);
}

// Randomized kind: the in-register radix-2 stages over element bits 0..3.
__device__ __forceinline__ void rand_stages_in_chunk(float v[kChunk]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      if ((e >> b) & 1) continue;
      const float a = v[e], d = v[e | (1 << b)];
      v[e] = a + d;
      v[e | (1 << b)] = a - d;
    }
  }
}

// Randomized kind: the radix-2 stages over lane bits 0..LOG2G-5 of one value.
template <int LOG2G>
__device__ __forceinline__ float rand_stages_across_lanes(float x, int lane) {
  if constexpr (LOG2G >= 5) x = bfly2_lanes<1>(x, lane);
  if constexpr (LOG2G >= 6) x = bfly2_lanes<2>(x, lane);
  if constexpr (LOG2G >= 7) x = bfly2_lanes<4>(x, lane);
  if constexpr (LOG2G >= 8) x = bfly2_lanes<8>(x, lane);
  if constexpr (LOG2G >= 9) x = bfly2_lanes<16>(x, lane);
  if constexpr (LOG2G >= 10) x = bfly2_lanes<32>(x, lane);
  return x;
}

// Regular kind: base-4 digit 0 (element bits 0-1) in registers.
__device__ __forceinline__ void regular_digit0(float v[kChunk]) {
#pragma unroll
  for (int a = 0; a < 4; ++a) bfly4(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
}

// Regular kind: base-4 digit 1 (element bits 2-3) in registers.
__device__ __forceinline__ void regular_digit1(float v[kChunk]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) bfly4(v[b], v[4 + b], v[8 + b], v[12 + b]);
}

// Scale that turns the unnormalised transform into the orthonormal one:
// 2^-(LOG2G/2) for the regular kind (one factor 1/2 per radix-4 stage),
// 1/sqrt(G) for the randomized kind.
template <int LOG2G, bool RAND>
__device__ __forceinline__ float rot_norm() {
  return RAND ? (1.0f / __builtin_sqrtf(static_cast<float>(1 << LOG2G))) : __builtin_ldexpf(1.0f, -(LOG2G / 2));
}

// The whole unnormalised rotation of one chunk per lane (randomized kind:
// with the chunk's sign words from load_signs), for a group size
// G = 2^log2g known only at run time (a uniform branch per stage): the
// steps above in the pack kernel's order, so the values are the pack
// kernel's bit for bit.
template <bool RAND>
__device__ __forceinline__ void rotate_chunk(float v[kChunk], int lane, int log2g, u32x4 signs) {
  if constexpr (RAND) {
    apply_sign_words(signs, v);
    rand_stages_in_chunk(v);
    // one stage at a time over all elements (each element still takes the
    // stages in the pack kernel's order)
    auto stage = [&](auto mask_c) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) v[e] = bfly2_lanes<decltype(mask_c)::value>(v[e], lane);
    };
    if (log2g >= 5) stage(std::integral_constant<int, 1>{});
    if (log2g >= 6) stage(std::integral_constant<int, 2>{});
    if (log2g >= 7) stage(std::integral_constant<int, 4>{});
    if (log2g >= 8) stage(std::integral_constant<int, 8>{});
    if (log2g >= 9) stage(std::integral_constant<int, 16>{});
    if (log2g >= 10) stage(std::integral_constant<int, 32>{});
  } else {
    regular_digit0(v);
    if (log2g >= 4) regular_digit1(v);
    if (log2g >= 6) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) v[e] = bfly4_lanes<0>(v[e]);
    }
    if (log2g >= 8) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) v[e] = bfly4_lanes<1>(v[e]);
    }
    if (log2g >= 10) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) v[e] = bfly4_lanes<2>(v[e]);
    }
  }
}

// rot_norm for a group size known only at run time: the same compile-time
// constants (a run-time square root need not round like the constant one).
__device__ __forceinline__ float rot_norm_rt(int log2g, bool rand) {
  if (rand) {
    switch (log2g) {
      case 4: return rot_norm<4, true>();
      case 5: return rot_norm<5, true>();
      case 6: return rot_norm<6, true>();
      case 7: return rot_norm<7, true>();
      case 8: return rot_norm<8, true>();
      case 9: return rot_norm<9, true>();
      default: return rot_norm<10, true>();
    }
  }
  switch (log2g) {
    case 2: return rot_norm<2, false>();
    case 4: return rot_norm<4, false>();
    case 6: return rot_norm<6, false>();
    case 8: return rot_norm<8, false>();
    default: return rot_norm<10, false>();
  }
}

// Largest magnitude of a chunk's values (the per-lane part of the row max).
__device__ __forceinline__ float chunk_absmax(const float v[kChunk], float m) {
#pragma unroll
  for (int e = 0; e < kChunk; e += 2) m = fmaxf(m, fmaxf(fabsf(v[e]), fabsf(v[e + 1])));
  return m;
}

// Round-to-nearest-even int8 codes of a*inv..d*inv (|.| <= 127 + tiny),
// packed little-endian into one dword.
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: ulp 1, low byte = two's complement code
  const uint32_t qa = as_u(fmaf(a, inv, kMagic));
  const uint32_t qb = as_u(fmaf(b, inv, kMagic));
  const uint32_t qc = as_u(fmaf(c, inv, kMagic));
  const uint32_t qd = as_u(fmaf(d, inv, kMagic));
  const uint32_t ab = __builtin_amdgcn_perm(qb, qa, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(qd, qc, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// The 16 int8 codes of a chunk, one 16-byte vector.
__device__ __forceinline__ u32x4 quant_chunk(const float v[kChunk], float inv) {
  u32x4 o;
  o.x = quant4(v[0], v[1], v[2], v[3], inv);
  o.y = quant4(v[4], v[5], v[6], v[7], inv);
  o.z = quant4(v[8], v[9], v[10], v[11], inv);
  o.w = quant4(v[12], v[13], v[14], v[15], inv);
  return o;
}

// Sixteen codes of one chunk as int4 nibble pairs (element 2j in the low,
// 2j + 1 in the high nibble of byte j): the even and the odd codes are each
// gathered into a dword of bytes by quant4, and one bit-field insert merges
// their low nibbles.  |code| <= 7, so the low nibble of a code's byte is its
// 4-bit two's complement.
__device__ __forceinline__ uint32_t quant8_nibbles(const float* v, float inv) {
  const uint32_t even = quant4(v[0], v[2], v[4], v[6], inv);
  const uint32_t odd = quant4(v[1], v[3], v[5], v[7], inv);
  return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

// The row's unnormalised maximum amax_u turned into the quantisation
// factor qmax / amax_u (0 for an all-zero row) and the row's scale
// amax_u * norm / qmax.
__device__ __forceinline__ float quant_factor(float amax_u, float qmax) { return amax_u > 0.f ? qmax / amax_u : 0.f; }
__device__ __forceinline__ float row_scale(float amax_u, float norm, float qmax) { return (amax_u * norm) / qmax; }

}  // namespace pack
}  // namespace convrot
