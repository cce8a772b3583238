// Fused group rotation + row absmax + int8 quantisation ("pack") for gfx950.
//
// What it computes ("INT8 Convrot Safetensors", sections "How INT8 convrot
// works", "Weight quantization", "Runtime activation quantization"): every
// contiguous group of G features of a row is multiplied by R_G, the
// normalised Kronecker power of the 4x4 regular Hadamard matrix H4; the
// row's scale is its largest rotated magnitude over 127; codes are the
// rotated values divided by the scale, rounded to nearest (ties to even) and
// clamped to [-127, 127].  The randomized kind ("Add experimental W8A8 MatMul
// with optional QuaRot-style rotation", section "Rotation method") multiplies
// each block by fixed +-1 signs, applies the natural-order Walsh-Hadamard
// transform and scales by 1/sqrt(G).  The int4 weight mode
// (stable-diffusion.cpp PR "load ConvRot int4 and per-channel int8
// safetensors", sections "Solution" and "The rotation") takes the largest
// rotated magnitude over 7, clamps to [-7, 7] and packs adjacent codes into
// the low and high nibble of one byte.
//
// Design (one workgroup per row, the whole row held in VGPRs):
//  * Each thread owns 1, 2 or 4 chunks of 16 contiguous features (two
//    16-byte loads per chunk for bf16, four for fp32), so one chunk's codes
//    are exactly one 16-byte store.  A G-group spans G/16 lanes of one
//    wavefront.  Rows are accessed through buffer resources sized to the
//    row: loads past K return zeros and stores past K are dropped.
//  * H4 = J/2 - (anti-diagonal), so an in-register radix-4 butterfly on
//    (a0..a3) is s = a0+a1+a2+a3, y_j = s - 2 a_{3-j} (3 adds + 4 FMAs).  The
//    factor 1/2 of every stage is left out and the total power of two is
//    folded into the scale at the end, which is bit-identical (binary
//    scaling commutes with fp32 rounding).
//  * The two low base-4 digits of a group index live inside a chunk
//    (in-register butterflies).  Higher digits live in lane bits.  With the
//    partner lane holding digit 3 - d, y_d = (a_d - a_{3-d}) + (sum of the
//    other pair): three two-operand instructions per element, each taking
//    its lane exchange as a DPP source (quad_perm within 4 lanes, row_ror
//    within 16), or ds_swizzle / a 32-lane exchange for G = 1024.  The digit
//    held in lane bits 2-3 (and 4-5) is Gray-coded across lanes, so that the
//    partner holding digit 3-j is always lane ^ 8 (or lane ^ 32).
//  * Absmax: per-thread max, then an unsigned max over the bit patterns of
//    the (non-negative) per-lane maxima across the wavefront, then LDS
//    across wavefronts.  Quantisation multiplies by 127/amax and rounds with
//    the 1.5*2^23 trick (one FMA rounds to nearest even and leaves the int8
//    code in the low byte); three v_perm_b32 pack four codes per dword.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lanes.h"
#include "launchers.h"

namespace convrot {
namespace {

constexpr int kChunk = 16;
constexpr int kMaxThreads = 1024;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

using namespace lanes;

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

// Position of a lane's chunk inside its group.  Regular kind: base-4 digit
// 0 of the lane position as is, digits 1 and 2 Gray-coded.  Randomized kind:
// identity (radix-2 exchanges need no reordering).
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

template <>
__device__ __forceinline__ void load_chunk<uint16_t>(__amdgpu_buffer_rsrc_t r, int elem_off, float v[kChunk]) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * elem_off, 0, kNonTemporal);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, 2 * elem_off + 16, 0, kNonTemporal);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = as_f(w[i] << 16);
    v[2 * i + 1] = as_f(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load_chunk<float>(__amdgpu_buffer_rsrc_t r, int elem_off, float v[kChunk]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, 4 * elem_off + 16 * i, 0, kNonTemporal);
    v[4 * i] = as_f(a.x); v[4 * i + 1] = as_f(a.y); v[4 * i + 2] = as_f(a.z); v[4 * i + 3] = as_f(a.w);
  }
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

// QMODE: 0 rotation only (fp32 rows to xrot), 1 int8 codes, 2 int4 codes
// (nibble pairs, K / 2 bytes per row, scale = max / 7).
// PRE (int8 codes, regular kind): the row maximum comes from `pmax`
// [rows, ldp], the largest magnitude of every G-group of the row's rotated
// values as a producing layer's epilogue computed it with the same
// operations (lanes.h); every wavefront takes the maximum of those K / G
// values itself, so the row needs no exchange between wavefronts.
template <typename InT, int LOG2G, bool RAND, int QMODE, int CPT, bool PRE = false>
__global__ __launch_bounds__(kMaxThreads) void pack_rows_kernel(
    const InT* __restrict__ X, int64_t ldx, int K, const int8_t* __restrict__ signs,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale,
    float* __restrict__ xrot, int64_t ldr, const float* __restrict__ pmax, int64_t ldp) {
  static_assert(!PRE || (QMODE == 1 && !RAND), "given group maxima: int8 codes of the regular kind");
  constexpr int G = 1 << LOG2G;
  constexpr int L = G >= kChunk ? G / kChunk : 1;  // lanes per group
  static_assert(L <= 64, "a group must fit in one wavefront");
  static_assert(RAND ? (LOG2G >= 4 && LOG2G <= 10) : (LOG2G % 2 == 0 && LOG2G >= 2 && LOG2G <= 10),
                "unsupported group size");
  __shared__ uint32_t wave_amax[kMaxThreads / 64];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int T = blockDim.x;
  const int lane = tid & 63;
  const InT* xrow = X + static_cast<int64_t>(row) * ldx;

  // Given group maxima: the row's maximum of them, requested before the
  // row itself so that the two loads overlap (one value live, not the row).
  uint32_t pre_bits = 0;
  if constexpr (PRE) {
    // through a buffer resource sized to the row's K / G maxima: reads past
    // the end return 0, so the loop is uniform and needs no lane test
    const int ngroups = K >> LOG2G;
    const __amdgpu_buffer_rsrc_t pr = row_rsrc(pmax + static_cast<int64_t>(row) * ldp, 4 * ngroups);
    for (int g0 = 0; g0 < ngroups; g0 += 64)
      pre_bits = max(pre_bits, static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(pr, 4 * (g0 + lane), 0, 0)));
  }

  const __amdgpu_buffer_rsrc_t xr = row_rsrc(xrow, K * static_cast<int>(sizeof(InT)));
  float v[CPT][kChunk];
  int off[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int vt = tid + c * T;
    const int grp = vt / L;
    const int pos = vt % L;
    off[c] = (grp * L + chunk_in_group<RAND>(pos)) * kChunk;
    load_chunk<InT>(xr, off[c], v[c]);
  }

  if constexpr (RAND) {
    const __amdgpu_buffer_rsrc_t sr = row_rsrc(signs, K);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const u32x4 sv = __builtin_amdgcn_raw_buffer_load_b128(sr, off[c], 0, 0);
      const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        const int8_t sgn = static_cast<int8_t>((w[e >> 2] >> (8 * (e & 3))) & 0xFF);
        v[c][e] = sgn < 0 ? -v[c][e] : v[c][e];
      }
    }
    // In-register radix-2 stages over element bits 0..3.
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          if ((e >> b) & 1) continue;
          const float a = v[c][e], d = v[c][e | (1 << b)];
          v[c][e] = a + d;
          v[c][e | (1 << b)] = a - d;
        }
      }
    }
    // Lane bits 0..LOG2G-5.
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        float x = v[c][e];
        if constexpr (LOG2G >= 5) x = bfly2_lanes<1>(x, lane);
        if constexpr (LOG2G >= 6) x = bfly2_lanes<2>(x, lane);
        if constexpr (LOG2G >= 7) x = bfly2_lanes<4>(x, lane);
        if constexpr (LOG2G >= 8) x = bfly2_lanes<8>(x, lane);
        if constexpr (LOG2G >= 9) x = bfly2_lanes<16>(x, lane);
        if constexpr (LOG2G >= 10) x = bfly2_lanes<32>(x, lane);
        v[c][e] = x;
      }
    }
  } else {
    // Base-4 digit 0 (element bits 0-1), in registers.
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int a = 0; a < 4; ++a) bfly4(v[c][4 * a], v[c][4 * a + 1], v[c][4 * a + 2], v[c][4 * a + 3]);
    }
    // Digit 1 (element bits 2-3), in registers.
    if constexpr (LOG2G >= 4) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
#pragma unroll
        for (int b = 0; b < 4; ++b) bfly4(v[c][b], v[c][4 + b], v[c][8 + b], v[c][12 + b]);
      }
    }
    // Digits 2.. across lanes, one digit at a time over all elements (the
    // independent elements fill the wait states a DPP read needs after the
    // write of its source).
    auto lane_stage = [&](auto k_c) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int e = 0; e < kChunk; ++e) v[c][e] = bfly4_lanes<decltype(k_c)::value>(v[c][e]);
    };
    if constexpr (LOG2G >= 6) lane_stage(std::integral_constant<int, 0>{});
    if constexpr (LOG2G >= 8) lane_stage(std::integral_constant<int, 1>{});
    if constexpr (LOG2G >= 10) lane_stage(std::integral_constant<int, 2>{});
  }

  // Scale that turns the unnormalised transform into the orthonormal one:
  // 2^-(LOG2G/2) for the regular kind (one factor 1/2 per radix-4 stage),
  // 1/sqrt(G) for the randomized kind.
  const float norm = RAND ? (1.0f / __builtin_sqrtf(static_cast<float>(G)))
                          : __builtin_ldexpf(1.0f, -(LOG2G / 2));

  if constexpr (QMODE == 0) {
    const __amdgpu_buffer_rsrc_t rr = row_rsrc(xrot + static_cast<int64_t>(row) * ldr, 4 * K);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 o = {v[c][4 * i] * norm, v[c][4 * i + 1] * norm, v[c][4 * i + 2] * norm, v[c][4 * i + 3] * norm};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rr, 4 * off[c] + 16 * i, 0, 0);
      }
    }
    return;
  } else {
    float amax_u;
    if constexpr (PRE) {
      // The given maxima are of the normalised values; norm is a power of
      // two, so dividing it out again is exact.  The lane's own maximum is
      // still formed (and kept by an empty asm use): without a use of every
      // rotated value right after the rotation, the compiler interleaves
      // the rotation with the quantisation and four chunks per thread no
      // longer fit the registers of a 1024-thread workgroup (measured: 75
      // spilled registers and a 4x slower launch).
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
#pragma unroll
        for (int e = 0; e < kChunk; e += 2) m = fmaxf(m, fmaxf(fabsf(v[c][e]), fabsf(v[c][e + 1])));
      }
      asm volatile("" ::"v"(m));
      amax_u = as_f(wave_max_bits(pre_bits)) / norm;
    } else {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
#pragma unroll
        for (int e = 0; e < kChunk; e += 2) m = fmaxf(m, fmaxf(fabsf(v[c][e]), fabsf(v[c][e + 1])));
      }
      // Every lane ends with its wavefront's maximum; rows of several
      // wavefronts combine theirs through LDS (uniform branch: T is the
      // workgroup size).
      uint32_t amax_bits = wave_max_bits(as_u(m));
      const int nwaves = T >> 6;
      if (nwaves > 1) {
        if (lane == 0) wave_amax[tid >> 6] = amax_bits;
        __syncthreads();
        amax_bits = wave_amax[0];
        for (int w = 1; w < nwaves; ++w) amax_bits = max(amax_bits, wave_amax[w]);
      }
      amax_u = as_f(amax_bits);
    }

    // Unnormalised codes: y_u * (qmax / amax_u) == y / s exactly up to the
    // rounding of the reciprocal; all-zero rows give inv = 0 and codes 0.
    constexpr float kQMax = QMODE == 2 ? 7.0f : 127.0f;
    const float inv = amax_u > 0.f ? kQMax / amax_u : 0.f;
    if (tid == 0) scale[row] = (amax_u * norm) / kQMax;

    if constexpr (QMODE == 1) {
      const __amdgpu_buffer_rsrc_t qr = row_rsrc(q + static_cast<int64_t>(row) * ldq, K);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        u32x4 o;
        o.x = quant4(v[c][0], v[c][1], v[c][2], v[c][3], inv);
        o.y = quant4(v[c][4], v[c][5], v[c][6], v[c][7], inv);
        o.z = quant4(v[c][8], v[c][9], v[c][10], v[c][11], inv);
        o.w = quant4(v[c][12], v[c][13], v[c][14], v[c][15], inv);
        __builtin_amdgcn_raw_buffer_store_b128(o, qr, off[c], 0, kNonTemporal);
      }
    } else {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const __amdgpu_buffer_rsrc_t qr = row_rsrc(q + static_cast<int64_t>(row) * ldq, K / 2);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const u32x2 o = {quant8_nibbles(&v[c][0], inv), quant8_nibbles(&v[c][8], inv)};
        __builtin_amdgcn_raw_buffer_store_b64(o, qr, off[c] / 2, 0, kNonTemporal);
      }
    }
  }
}

template <typename InT, int LOG2G, bool RAND, int QMODE, bool PRE = false>
hipError_t dispatch_cpt(const void* X, int64_t rows, int64_t K, int64_t ldx, const int8_t* signs,
                        int8_t* q, int64_t ldq, float* scale, float* xrot, int64_t ldr,
                        hipStream_t stream, const float* pmax = nullptr, int64_t ldp = 0) {
  const int64_t nvt = K / kChunk;  // chunks in a row
  // Chunks per thread: more of them spread the per-wavefront fixed work (the
  // reductions, the scale division, addressing) over more elements; take 2
  // or 4 while the row keeps at least two whole wavefronts (one wavefront
  // per row was measured slower: less parallelism per row), and as many as
  // needed to stay within one workgroup.
  int cpt = 1;
  while (cpt < 4 && nvt % (128 * cpt) == 0) cpt *= 2;
  while ((nvt + cpt - 1) / cpt > kMaxThreads) cpt *= 2;
  const int64_t threads = ((nvt + cpt - 1) / cpt + 63) / 64 * 64;
  const dim3 grid(static_cast<unsigned>(rows));
  const dim3 block(static_cast<unsigned>(threads));
  const InT* x = static_cast<const InT*>(X);
  switch (cpt) {
    case 1:
      hipLaunchKernelGGL((pack_rows_kernel<InT, LOG2G, RAND, QMODE, 1, PRE>), grid, block, 0, stream, x, ldx,
                         static_cast<int>(K), signs, q, ldq, scale, xrot, ldr, pmax, ldp);
      break;
    case 2:
      hipLaunchKernelGGL((pack_rows_kernel<InT, LOG2G, RAND, QMODE, 2, PRE>), grid, block, 0, stream, x, ldx,
                         static_cast<int>(K), signs, q, ldq, scale, xrot, ldr, pmax, ldp);
      break;
    case 4:
      hipLaunchKernelGGL((pack_rows_kernel<InT, LOG2G, RAND, QMODE, 4, PRE>), grid, block, 0, stream, x, ldx,
                         static_cast<int>(K), signs, q, ldq, scale, xrot, ldr, pmax, ldp);
      break;
    default:
      return hipErrorInvalidValue;  // K above 64 * 1024 is rejected by the caller
  }
  return hipGetLastError();
}

template <typename InT, bool RAND, int QMODE>
hipError_t dispatch_group(int log2G, const void* X, int64_t rows, int64_t K, int64_t ldx,
                          const int8_t* signs, int8_t* q, int64_t ldq, float* scale, float* xrot,
                          int64_t ldr, hipStream_t stream) {
#define CONVROT_PACK_CASE(LG)                                                                   \
  case LG:                                                                                      \
    return dispatch_cpt<InT, LG, RAND, QMODE>(X, rows, K, ldx, signs, q, ldq, scale, xrot, ldr, \
                                              stream);
  if constexpr (RAND) {
    switch (log2G) {
      CONVROT_PACK_CASE(4)
      CONVROT_PACK_CASE(5)
      CONVROT_PACK_CASE(6)
      CONVROT_PACK_CASE(7)
      CONVROT_PACK_CASE(8)
      CONVROT_PACK_CASE(9)
      CONVROT_PACK_CASE(10)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (log2G) {
      CONVROT_PACK_CASE(2)
      CONVROT_PACK_CASE(4)
      CONVROT_PACK_CASE(6)
      CONVROT_PACK_CASE(8)
      CONVROT_PACK_CASE(10)
      default: return hipErrorInvalidValue;
    }
  }
#undef CONVROT_PACK_CASE
}

template <typename InT, int QMODE>
hipError_t dispatch_kind(int log2G, RotKind kind, const void* X, int64_t rows, int64_t K, int64_t ldx,
                         const int8_t* signs, int8_t* q, int64_t ldq, float* scale, float* xrot, int64_t ldr,
                         hipStream_t stream) {
  if (kind == RotKind::Randomized)
    return dispatch_group<InT, true, QMODE>(log2G, X, rows, K, ldx, signs, q, ldq, scale, xrot, ldr, stream);
  return dispatch_group<InT, false, QMODE>(log2G, X, rows, K, ldx, signs, q, ldq, scale, xrot, ldr, stream);
}

template <int QMODE>
hipError_t dispatch_input(Elt xdt, int log2G, RotKind kind, const void* X, int64_t rows, int64_t K, int64_t ldx,
                          const int8_t* signs, int8_t* q, int64_t ldq, float* scale, float* xrot, int64_t ldr,
                          hipStream_t stream) {
  if (xdt == Elt::BF16)
    return dispatch_kind<uint16_t, QMODE>(log2G, kind, X, rows, K, ldx, signs, q, ldq, scale, xrot, ldr, stream);
  return dispatch_kind<float, QMODE>(log2G, kind, X, rows, K, ldx, signs, q, ldq, scale, xrot, ldr, stream);
}

template <typename InT>
hipError_t dispatch_prescaled(int log2G, const void* X, int64_t rows, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                              float* scale, const float* pmax, int64_t ldp, hipStream_t stream) {
#define CONVROT_PRE_CASE(LG)                                                                                 \
  case LG:                                                                                                   \
    return dispatch_cpt<InT, LG, false, 1, true>(X, rows, K, ldx, nullptr, q, ldq, scale, nullptr, 0, stream, \
                                                 pmax, ldp);
  switch (log2G) {
    CONVROT_PRE_CASE(2)
    CONVROT_PRE_CASE(4)
    CONVROT_PRE_CASE(6)
    CONVROT_PRE_CASE(8)
    default: return hipErrorInvalidValue;  // G = 1024 cannot come from a 256-wide producing tile
  }
#undef CONVROT_PRE_CASE
}

}  // namespace

hipError_t launch_pack_rows_prescaled(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                                      const float* pmax, int64_t ldp, int8_t* q, int64_t ldq, float* scale,
                                      hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (xdt == Elt::BF16)
    return dispatch_prescaled<uint16_t>(log2G, X, rows, K, ldx, q, ldq, scale, pmax, ldp, stream);
  return dispatch_prescaled<float>(log2G, X, rows, K, ldx, q, ldq, scale, pmax, ldp, stream);
}

hipError_t launch_pack_rows(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                            RotKind kind, const int8_t* signs, int8_t* q, int64_t ldq, float* scale,
                            float* xrot, int64_t ldr, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (q != nullptr)
    return dispatch_input<1>(xdt, log2G, kind, X, rows, K, ldx, signs, q, ldq, scale, nullptr, 0, stream);
  return dispatch_input<0>(xdt, log2G, kind, X, rows, K, ldx, signs, nullptr, 0, scale, xrot, ldr, stream);
}

hipError_t launch_pack_rows_w4(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                               RotKind kind, const int8_t* signs, uint8_t* q, int64_t ldq, float* scale,
                               hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return dispatch_input<2>(xdt, log2G, kind, X, rows, K, ldx, signs, reinterpret_cast<int8_t*>(q), ldq, scale,
                           nullptr, 0, stream);
}

}  // namespace convrot
