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

#include "launchers.h"
#include "pack_core.h"

namespace convrot {
namespace {

constexpr int kMaxThreads = 1024;

using namespace pack;

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
    int8_t* __restrict__ q, int64_t ldq, bool t16, float* __restrict__ scale,
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

  // The steps of pack_core.h, each over all of the thread's chunks.
  if constexpr (RAND) {
    const __amdgpu_buffer_rsrc_t sr = row_rsrc(signs, K);
#pragma unroll
    for (int c = 0; c < CPT; ++c) apply_signs(sr, off[c], v[c]);
#pragma unroll
    for (int c = 0; c < CPT; ++c) rand_stages_in_chunk(v[c]);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) v[c][e] = rand_stages_across_lanes<LOG2G>(v[c][e], lane);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c) regular_digit0(v[c]);
    if constexpr (LOG2G >= 4) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) regular_digit1(v[c]);
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

  const float norm = rot_norm<LOG2G, RAND>();

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
      for (int c = 0; c < CPT; ++c) m = chunk_absmax(v[c], m);
      asm volatile("" ::"v"(m));
      amax_u = as_f(wave_max_bits(pre_bits)) / norm;
    } else {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) m = chunk_absmax(v[c], m);
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
    const float inv = quant_factor(amax_u, kQMax);
    if (tid == 0) scale[row] = row_scale(amax_u, norm, kQMax);

    if constexpr (QMODE == 1) {
      // t16 (TILE16 codes, ldq == K, K % 64 == 0): byte b of the row lies at
      // (b / 64) KiB + (row % 16) 64 + b % 64 from its 16-row tile.
      const int64_t base = t16 ? (row >> 4) * 16 * ldq + (row & 15) * 64 : static_cast<int64_t>(row) * ldq;
      const __amdgpu_buffer_rsrc_t qr = row_rsrc(q + base, t16 ? (K >> 6) << 10 : K);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int o = t16 ? ((off[c] >> 6) << 10) | (off[c] & 63) : off[c];
        __builtin_amdgcn_raw_buffer_store_b128(quant_chunk(v[c], inv), qr, o, 0, kNonTemporal);
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
                        int8_t* q, int64_t ldq, bool t16, float* scale, float* xrot, int64_t ldr,
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
                         static_cast<int>(K), signs, q, ldq, t16, scale, xrot, ldr, pmax, ldp);
      break;
    case 2:
      hipLaunchKernelGGL((pack_rows_kernel<InT, LOG2G, RAND, QMODE, 2, PRE>), grid, block, 0, stream, x, ldx,
                         static_cast<int>(K), signs, q, ldq, t16, scale, xrot, ldr, pmax, ldp);
      break;
    case 4:
      hipLaunchKernelGGL((pack_rows_kernel<InT, LOG2G, RAND, QMODE, 4, PRE>), grid, block, 0, stream, x, ldx,
                         static_cast<int>(K), signs, q, ldq, t16, scale, xrot, ldr, pmax, ldp);
      break;
    default:
      return hipErrorInvalidValue;  // K above 64 * 1024 is rejected by the caller
  }
  return hipGetLastError();
}

template <typename InT, bool RAND, int QMODE>
hipError_t dispatch_group(int log2G, const void* X, int64_t rows, int64_t K, int64_t ldx,
                          const int8_t* signs, int8_t* q, int64_t ldq, bool t16, float* scale, float* xrot,
                          int64_t ldr, hipStream_t stream) {
#define CONVROT_PACK_CASE(LG)                                                                        \
  case LG:                                                                                           \
    return dispatch_cpt<InT, LG, RAND, QMODE>(X, rows, K, ldx, signs, q, ldq, t16, scale, xrot, ldr, \
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
                         const int8_t* signs, int8_t* q, int64_t ldq, bool t16, float* scale, float* xrot,
                         int64_t ldr, hipStream_t stream) {
  if (kind == RotKind::Randomized)
    return dispatch_group<InT, true, QMODE>(log2G, X, rows, K, ldx, signs, q, ldq, t16, scale, xrot, ldr, stream);
  return dispatch_group<InT, false, QMODE>(log2G, X, rows, K, ldx, signs, q, ldq, t16, scale, xrot, ldr, stream);
}

template <int QMODE>
hipError_t dispatch_input(Elt xdt, int log2G, RotKind kind, const void* X, int64_t rows, int64_t K, int64_t ldx,
                          const int8_t* signs, int8_t* q, int64_t ldq, bool t16, float* scale, float* xrot,
                          int64_t ldr, hipStream_t stream) {
  if (xdt == Elt::BF16)
    return dispatch_kind<uint16_t, QMODE>(log2G, kind, X, rows, K, ldx, signs, q, ldq, t16, scale, xrot, ldr,
                                          stream);
  return dispatch_kind<float, QMODE>(log2G, kind, X, rows, K, ldx, signs, q, ldq, t16, scale, xrot, ldr, stream);
}

template <typename InT>
hipError_t dispatch_prescaled(int log2G, const void* X, int64_t rows, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                              float* scale, const float* pmax, int64_t ldp, hipStream_t stream) {
#define CONVROT_PRE_CASE(LG)                                                                                 \
  case LG:                                                                                                   \
    return dispatch_cpt<InT, LG, false, 1, true>(X, rows, K, ldx, nullptr, q, ldq, false, scale, nullptr, 0, \
                                                 stream, pmax, ldp);
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
                            float* xrot, int64_t ldr, hipStream_t stream, bool t16) {
  if (rows == 0) return hipSuccess;
  if (q != nullptr)
    return dispatch_input<1>(xdt, log2G, kind, X, rows, K, ldx, signs, q, ldq, t16, scale, nullptr, 0, stream);
  return dispatch_input<0>(xdt, log2G, kind, X, rows, K, ldx, signs, nullptr, 0, false, scale, xrot, ldr, stream);
}

hipError_t launch_pack_rows_w4(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                               RotKind kind, const int8_t* signs, uint8_t* q, int64_t ldq, float* scale,
                               hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return dispatch_input<2>(xdt, log2G, kind, X, rows, K, ldx, signs, reinterpret_cast<int8_t*>(q), ldq, false,
                           scale, nullptr, 0, stream);
}

}  // namespace convrot
