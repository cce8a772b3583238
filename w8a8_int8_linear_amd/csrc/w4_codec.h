// int4 weight codes in registers: nibble pairs -> int8 codes.
//
// Format (stable-diffusion.cpp PR "load ConvRot int4 and per-channel int8
// safetensors", sections "Solution" and "The rotation"): codes in [-7, 7],
// two per byte, element 2j in the low and 2j + 1 in the high nibble of byte
// j, each as 4-bit two's complement.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

typedef int w4_i32x4 __attribute__((ext_vector_type(4)));

// Each byte's nibble n (0..15) becomes the int8 (n ^ 8) - 8: n ^ 0x88 sets
// bit 7, so subtracting 8 never borrows from the next byte, and bit 7 is
// flipped back afterwards.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t b) {
  return ((b ^ 0x88888888u) - 0x08080808u) ^ 0x80808080u;
}

// 16 codes held in 8 bytes (w0 = bytes 0-3) -> 16 int8 codes in element
// order.  Per dword the low and the high nibbles are split into bytes and
// interleaved back with one byte permute each (perm(hi, lo, sel) takes bytes
// 0-3 from lo and 4-7 from hi).
__device__ __forceinline__ w4_i32x4 expand_w4(uint32_t w0, uint32_t w1) {
  const uint32_t lo0 = w0 & 0x0F0F0F0Fu, hi0 = (w0 >> 4) & 0x0F0F0F0Fu;
  const uint32_t lo1 = w1 & 0x0F0F0F0Fu, hi1 = (w1 >> 4) & 0x0F0F0F0Fu;
  return w4_i32x4{static_cast<int>(sext_nibbles(__builtin_amdgcn_perm(hi0, lo0, 0x05010400u))),
                  static_cast<int>(sext_nibbles(__builtin_amdgcn_perm(hi0, lo0, 0x07030602u))),
                  static_cast<int>(sext_nibbles(__builtin_amdgcn_perm(hi1, lo1, 0x05010400u))),
                  static_cast<int>(sext_nibbles(__builtin_amdgcn_perm(hi1, lo1, 0x07030602u)))};
}

}  // namespace convrot
