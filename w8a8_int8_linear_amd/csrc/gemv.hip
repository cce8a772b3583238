// Small-M (decode) linear for gfx950, bound by reading the weight once.
//
// int8 mode: exact int32 A = Qx Qw^T, then Y = A s_x[r] s_w[o] + b[o] ("INT8
// Convrot Safetensors", "Runtime activation quantization"); the same result
// bits as the tiled kernel.  bf16 mode: Y = X W^T + b with fp32 accumulation,
// the unquantised linear that layers with K % G != 0 keep (sglang PR 34581
// summary page, kitchen_int8 routing).
//
// With M <= 16 the time is the time to stream N*K weight bytes.  Every
// vector load of an MFMA operand touches 16 rows (16 cache lines), so the
// CU's memory pipeline, counted in lines, is what streams: the structure
// keeps the lines per MFMA low and many of them in flight.
//  * A workgroup computes one 16-feature tile, or two that share every
//    activation fragment (plain launches with at least four tiles per CU);
//    its waves (4, or 8 where a wave would stream more than 32 K units)
//    split K.
//  * A K unit is 64 bytes of each of the 16 weight rows: one
//    v_mfma_i32_16x16x64_i8 (or v_mfma_f32_16x16x32_bf16) per tile whose row
//    operand is the 16 weight rows (16 bytes per lane, straight from global
//    memory) and whose column operand is the activation rows (rows >= M
//    re-read the last row; their outputs are dropped).
//  * Loads come in double-buffered rounds: the next round is requested
//    before the current one is multiplied.
//  * Where a wave streams at least five K units, each weight row's 128-byte
//    line goes global -> LDS whole (global_load_lds_dwordx4, 8 rows per
//    transfer, chunks XOR-swizzled by row) and the MFMA fragments are read
//    from LDS, so a line is touched once instead of twice (int8 weights in
//    the row layout, int4 weights with K % 32 == 0, and the 16-wave
//    workgroups below).  int8 TILE16 weights skip it: a wave's register
//    load of one unit already reads 1 KiB of consecutive memory.
//  * The partial accumulators of the waves are summed through LDS (exact in
//    int8 mode) and wave 0 applies the epilogue, writing 4 consecutive
//    outputs per lane.
//  * Fused epilogues (int8 mode): an activation of Y (GELU, erf or tanh
//    form), or a gated pair Y = act(gate) * up where the workgroup streams
//    the same 16 features of both weights against one set of activation
//    loads.
//  * When there are fewer 16-feature tiles than CUs (a down projection has
//    N = 1152, i.e. 72 tiles) and the caller supplies a workspace, K is also
//    split across workgroups: each (tile, K range) workgroup stores its
//    partial sums (exact int32 in int8 mode) in that workspace, and a second
//    launch of one wave per tile adds them in K order and applies the
//    epilogue.  The launch boundary makes the partials visible; inside one
//    launch that would take device-scope fences, which on this multi-XCD GPU
//    write back and invalidate a whole L2 each.  Same result bits as the
//    unsplit kernel in int8 mode.
//  * Plain int8 launches with at most 12 activation rows and fewer tiles
//    than CUs take neither: one workgroup of 16 waves per tile splits all
//    of K among its waves and adds through LDS, one launch (see
//    wide_tiles).
//  * TILE16 weights (convrot_tile_weight): the 16 rows of a tile store each
//    64-byte K unit as 1 KiB of consecutive memory; only the addresses of
//    the weight loads change.
//  * Launches that pack their own input (XP; convrot_linear_packin and
//    _gated_packin, up to 4 bf16 rows): each workgroup first packs the rows
//    into LDS with the pack kernel's steps (pack_core.h) while its first
//    weight rounds are in flight, then reads every activation fragment from
//    LDS.  Same codes, scales and result bits as packing first.
//  * int4 weights (W4A8; stable-diffusion.cpp PR "load ConvRot int4 and
//    per-channel int8 safetensors", sections "Solution" and "The rotation":
//    codes in [-7, 7], one scale per output row, adjacent pairs in a byte):
//    a K unit is 128 codes, one 16-byte load per lane and tile (half the
//    int8 lines per MFMA), expanded in registers to the int8 codes of two
//    MFMAs; the accumulator and epilogue are unchanged.
// The assignment of k to (MFMA, lane) is the same for both operands, so each
// MFMA pairs matching k.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "epilogue.h"
#include "launchers.h"
#include "pack_core.h"
#include "w4_codec.h"

namespace convrot {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kStepBytes = 64;   // bytes of one weight row per step

template <bool I8>
struct Mma;

template <>
struct Mma<true> {
  using Acc = i32x4;
  static __device__ __forceinline__ Acc run(i32x4 w, i32x4 x, Acc c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, c, 0, 0, 0);
  }
};

template <>
struct Mma<false> {
  using Acc = f32x4;
  static __device__ __forceinline__ Acc run(i32x4 w, i32x4 x, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, x), c,
                                                   0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ bool vec_ok(const T* p) {
  return (reinterpret_cast<uintptr_t>(p) & (4 * sizeof(T) - 1)) == 0;
}

typedef __attribute__((address_space(3))) void* gemv_lds_ptr_t;

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds + 16 l.
__device__ __forceinline__ void gemv_dma16(const uint8_t* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (gemv_lds_ptr_t)lds, 16, 0, 0);
}
// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void gemv_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Split-K state of one launch: partials [tile][split][set][64 lanes] x 16
// bytes, `steps` K steps per split.
struct SplitArgs {
  i32x4* part;
  int splits;
  int steps;
};

// Activation rows a launch packs itself (XP): bf16 X [M, ldx elements],
// rotated with G = 2^log2g of the regular or randomized kind (K signs for
// the latter) and quantised with the pack kernel's steps (pack_core.h).
struct XPackArgs {
  const void* X;
  int64_t ldx;
  int log2g;
  int rand;
  const int8_t* signs;
};

// The XP prologue: every thread of the workgroup (T >= K / 16 of them)
// takes one 16-feature chunk of each row, in the pack kernel's lane order
// (G / 16 lanes per group, chunk_in_group): the loads of all M rows (and
// of the chunk's signs) are issued first, then each row is rotated and its
// wavefront maximum posted; after one barrier every row's maximum gives its
// scale s_x[r] and the 16 codes of the chunk go to `codes` (row pitch
// `pitch` bytes).  Chunks past K read zeros and write nothing.  Ends with a
// barrier.
template <bool RAND, int WAVES>
__device__ __forceinline__ void xpack_rows(const XPackArgs& xp, int M, int K, uint8_t* codes, int pitch, float* s_x,
                                           uint32_t* wmax) {
  static_assert(WAVES % 4 == 0, "wavefront maxima are read four at a time");
  using namespace pack;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int L = xp.log2g >= 4 ? 1 << (xp.log2g - 4) : 1;  // lanes per group
  const int off = ((tid / L) * L + chunk_in_group<RAND>(tid % L)) * kChunk;
  // Every load first, unconditionally (rows past M re-read row M - 1), so
  // that all of them are in flight together.
  u32x4 raw[kPackinMaxRows][2];
#pragma unroll
  for (int r = 0; r < kPackinMaxRows; ++r) {
    const __amdgpu_buffer_rsrc_t xr =
        row_rsrc(static_cast<const uint16_t*>(xp.X) + static_cast<int64_t>(min(r, M - 1)) * xp.ldx, 2 * K);
    raw[r][0] = __builtin_amdgcn_raw_buffer_load_b128(xr, 2 * off, 0, kNonTemporal);
    raw[r][1] = __builtin_amdgcn_raw_buffer_load_b128(xr, 2 * off + 16, 0, kNonTemporal);
  }
  u32x4 sv = {0, 0, 0, 0};
  if constexpr (RAND) sv = load_signs(row_rsrc(xp.signs, K), off);
  float v[kPackinMaxRows][kChunk];
#pragma unroll
  for (int r = 0; r < kPackinMaxRows; ++r) {
    if (r < M) {
      bf16_words_to_chunk(raw[r][0], raw[r][1], v[r]);
      rotate_chunk<RAND>(v[r], lane, xp.log2g, sv);
      const uint32_t bits = wave_max_bits(as_u(chunk_absmax(v[r], 0.f)));
      if (lane == 0) wmax[r * WAVES + wid] = bits;
    }
  }
  __syncthreads();
  const float norm = rot_norm_rt(xp.log2g, RAND);
#pragma unroll
  for (int r = 0; r < kPackinMaxRows; ++r) {
    if (r < M) {
      // the row's WAVES wavefront maxima, read as 16-byte vectors
      uint32_t amax_bits = 0;
#pragma unroll
      for (int w = 0; w < WAVES; w += 4) {
        const u32x4 m4 = *reinterpret_cast<const u32x4*>(wmax + r * WAVES + w);
        amax_bits = max(amax_bits, max(max(m4.x, m4.y), max(m4.z, m4.w)));
      }
      const float amax_u = as_f(amax_bits);
      if (tid == 0) s_x[r] = row_scale(amax_u, norm, 127.f);
      if (off < K)
        *reinterpret_cast<u32x4*>(codes + r * pitch + off) = quant_chunk(v[r], quant_factor(amax_u, 127.f));
    }
  }
  __syncthreads();
}

// The epilogue's per-row and per-feature operands of one lane (row
// m = lane & 15, features n0 + 4 (lane >> 4) + r), loaded by the epilogue
// wave before its main loop so that they arrive with the first weights
// instead of after the last MFMA (indexes clamped into the operands; lanes
// past M or N store nothing).
template <bool GATED>
struct EpiIn {
  float s_row;
  float sb[4], b[4];
  float sb2[GATED ? 4 : 1], b2[GATED ? 4 : 1];
};

template <bool I8, int OUT, bool GATED>
__device__ __forceinline__ EpiIn<GATED> load_epi(int lane, int n0, const EpiArgs& epi, int M, int N) {
  EpiIn<GATED> in{};
  if constexpr (OUT != 2) {
    const int m = min(lane & 15, M - 1);
    const int n = n0 + 4 * (lane >> 4);
    in.s_row = I8 ? epi.sa[m] : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      in.sb[r] = I8 ? epi.sb[nn] : 1.f;
      in.b[r] = epi.bias ? epi.bias[nn] : 0.f;
      if constexpr (GATED) {
        in.sb2[r] = epi.sb2[nn];
        in.b2[r] = epi.bias2 ? epi.bias2[nn] : 0.f;
      }
    }
  }
  return in;
}

// Epilogue of one 16-feature tile: lane holds output row m = lane & 15 and
// features n0 + 4 (lane >> 4) + r of the accumulators acc[set].
template <bool I8, int OUT, int ACT, bool GATED, typename Acc>
__device__ __forceinline__ void tile_epilogue(const Acc* acc, int lane, int n0, const EpiIn<GATED>& in, int M,
                                              int N, void* __restrict__ C, int64_t ldc) {
  constexpr int kSets = GATED ? 2 : 1;
  const int m = lane & 15;
  const int n = n0 + 4 * (lane >> 4);
  if (m >= M || n >= N) return;
  if constexpr (OUT == 2) {
    int32_t* out = static_cast<int32_t*>(C) + static_cast<int64_t>(m) * ldc + n;
    if (n + 3 < N && vec_ok(out)) {
      *reinterpret_cast<i32x4*>(out) = __builtin_bit_cast(i32x4, acc[0]);
    } else {
      for (int r = 0; r < 4 && n + r < N; ++r) out[r] = acc[0][r];
    }
  } else {
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float b = in.b[r];
      y[r] = I8 ? fmaf(static_cast<float>(acc[0][r]), in.s_row * in.sb[r], b) : static_cast<float>(acc[0][r]) + b;
      if constexpr (GATED) {
        const float u = fmaf(static_cast<float>(acc[kSets - 1][r]), in.s_row * in.sb2[r], in.b2[r]);
        y[r] = activation<ACT>(y[r]) * u;
      } else {
        y[r] = activation<ACT>(y[r]);
      }
    }
    if constexpr (OUT == 0) {
      float* out = static_cast<float*>(C) + static_cast<int64_t>(m) * ldc + n;
      if (n + 3 < N && vec_ok(out)) {
        *reinterpret_cast<f32x4*>(out) = f32x4{y[0], y[1], y[2], y[3]};
      } else {
        for (int r = 0; r < 4 && n + r < N; ++r) out[r] = y[r];
      }
    } else {
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

// A: activation rows [M, lda bytes]; B: weight rows [N, ldb bytes] (int4
// mode: K / 2 bytes of nibble pairs per row); kbytes = K * element size of A
// (a multiple of 16); per = K units per wave.  A workgroup computes TILES
// consecutive 16-feature tiles that share each activation fragment.
//
// K unit: 64 activation bytes (one MFMA per tile), or in int4 mode 128 codes
// (two MFMAs per tile), where lane (row, ch) takes codes 32 ch .. 32 ch + 31
// of the unit from one 16-byte weight load (bytes 16 ch .. 16 ch + 15 of the
// unit's 64 nibble bytes) and two 16-byte activation loads; codes 0-15 of
// that range feed the first MFMA and 16-31 the second.  Both operands follow
// the same assignment of k to (MFMA, lane), so every product pairs matching
// k; the int32 sum does not depend on the order.
template <bool I8, int OUT, int WAVES, int ACT = 0, bool GATED = false, bool SPLIT = false, bool W4 = false,
          int TILES = 1, bool DMA = false, bool XP = false>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, EpiArgs epi, int M,
    int N_all, int kbytes, int per, void* __restrict__ C, int64_t ldc, SplitArgs sp, bool tiled, bool xtiled,
    XPackArgs xp) {
  static_assert(!GATED || I8, "the gated pair is an int8 feature");
  static_assert(!W4 || I8, "int4 weights pair with int8 activations");
  static_assert(TILES == 1 || (!GATED && !SPLIT), "several tiles per workgroup only on the plain unsplit path");
  static_assert(!XP || (I8 && !W4 && !SPLIT && TILES == 1), "a packing launch: int8 weights, one tile, no split");
  using Acc = typename Mma<I8>::Acc;
  constexpr int kSets = GATED ? 2 : 1;         // weight row sets streamed (gate, up)
  constexpr int kUnit = W4 ? 128 : kStepBytes;  // activation bytes per K unit
  constexpr int kRound = TILES == 1 ? 4 : 2;    // units per round of loads (two rounds in flight per wave)
  __shared__ Acc partial[kSets * TILES][WAVES > 1 ? WAVES - 1 : 1][64];
  static_assert(!DMA || I8, "LDS staging is for int8 and int4 weights");
  constexpr bool kDma = DMA;  // weights staged through LDS in whole lines
  __shared__ __attribute__((aligned(16))) uint8_t wring[kDma ? WAVES : 1][2][kDma ? kSets * TILES : 1][kDma ? 2048 : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  // The wide workgroups (16 waves, not packing) each take 8 output features:
  // rows 8-15 of the MFMA's weight operand repeat row 7 and their columns
  // are not written, which doubles the workgroups streaming a narrow
  // weight.  N below is this workgroup's end of the output features.
  constexpr bool kHalf = WAVES == 16 && !XP;
  const int n0 = kHalf ? blockIdx.x * 8 : blockIdx.x * 16 * TILES;
  const int N = kHalf ? min(N_all, n0 + 8) : N_all;
  const int row = lane & 15;
  const int ch = lane >> 4;

  // Weight rows: TILES tiles of each set; in int4 mode 16 nibble bytes per
  // lane and unit, else 16 weight bytes per lane and step.  A 64-byte unit
  // of a row lies unit_stride bytes after the previous one, and row r of a
  // tile row_pitch bytes after its first row: 64 and ldb in the row layout,
  // 1024 and 64 in the TILE16 layout (whose tiles start where the row
  // layout's 16-row blocks do, ldb being the bytes of one row; a workgroup
  // of 8 features may start in the middle of a tile).
  const int unit_stride = tiled ? 1024 : 64;
  const int64_t pitch1 = tiled ? 64 : ldb;
  const int64_t pitch2 = tiled ? 64 : epi.ldb2;
  const uint8_t* wrow[kSets][TILES];
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    const int64_t nt = n0 + 16 * i;
    const int64_t r = min(nt + row, static_cast<int64_t>(N) - 1) - nt;
    const int64_t tb = tiled ? (nt & ~int64_t{15}) : nt;
    const int64_t rr = tiled ? (nt & 15) + r : r;
    wrow[0][i] = B + tb * ldb + rr * pitch1 + ch * 16;
    if constexpr (GATED) wrow[kSets - 1][i] = epi.B2 + nt * epi.ldb2 + r * pitch2 + ch * 16;
  }
  // XP: the workgroup packs the M activation rows into LDS (codes at a
  // pitch of K + 16 bytes, then the row scales and the wavefront maxima;
  // the first round of weight transfers is issued before, so it lands
  // meanwhile), and every activation fragment is read from there.
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  typedef const __attribute__((address_space(3))) uint8_t* lds_bytes_t;
  typedef const __attribute__((address_space(3))) i32x4* lds_i32x4_t;
  const uint8_t* xrow = nullptr;
  lds_bytes_t xlds = nullptr;
  if constexpr (XP) {
    xlds = (lds_bytes_t)(xs + min(row, M - 1) * (kbytes + 16) + ch * 16);
  } else {
    // xtiled (int8 weights only): the activation rows in the TILE16 layout,
    // byte b of row r at (b / 64) KiB + r 64 + b % 64, so that a fragment
    // load of one unit reads 1 KiB of consecutive memory.
    xrow = A + (xtiled ? min(row, M - 1) * 64 : static_cast<int64_t>(min(row, M - 1)) * lda) + ch * (W4 ? 32 : 16);
  }
  auto xp_prologue = [&]() {
    if constexpr (XP) {
      const int pitch = kbytes + 16;
      float* s_x = reinterpret_cast<float*>(xs + M * pitch);
      uint32_t* wmax = reinterpret_cast<uint32_t*>(s_x + 4);
      if (xp.rand)
        xpack_rows<true, WAVES>(xp, M, kbytes, xs, pitch, s_x, wmax);
      else
        xpack_rows<false, WAVES>(xp, M, kbytes, xs, pitch, s_x, wmax);
      epi.sa = s_x;
    }
  };
  // 16 activation bytes of this lane at `byte` (LDS reads in XP launches,
  // so they never count against the vector-memory counter).
  auto xload = [&](int byte) -> i32x4 {
    if constexpr (XP)
      return *(lds_i32x4_t)(xlds + byte);
    else
      return *reinterpret_cast<const i32x4*>(xrow + (xtiled ? ((byte >> 6) << 10) + (byte & 63) : byte));
  };

  const int nunits = (kbytes + kUnit - 1) / kUnit;
  // K units [u_lo, u_hi) of this workgroup, `per` of them per wave.
  const int u_lo = SPLIT ? static_cast<int>(blockIdx.y) * sp.steps : 0;
  const int u_hi = SPLIT ? min(nunits, u_lo + sp.steps) : nunits;
  const int u_begin = u_lo + wid * per;
  const int u_end = min(u_hi, u_begin + per);

  EpiIn<GATED> epi_in[SPLIT ? 1 : TILES];
  auto load_epi_in = [&]() {
    if (!SPLIT && wid == 0) {
#pragma unroll
      for (int i = 0; i < (SPLIT ? 1 : TILES); ++i)
        epi_in[i] = load_epi<I8, OUT, GATED>(lane, n0 + 16 * i, epi, M, N);
    }
  };
  if constexpr (!XP) load_epi_in();  // XP: once the prologue has the row scales

  Acc acc[kSets][TILES];
#pragma unroll
  for (int t = 0; t < kSets; ++t)
#pragma unroll
    for (int i = 0; i < TILES; ++i) acc[t][i] = Acc{0, 0, 0, 0};
  // Rounds of kRound units, double-buffered: the loads of the next round are
  // issued before the MFMAs of the current one, so a wave keeps its weight
  // stream in flight while it multiplies.
  struct Round {
    i32x4 w[kSets][TILES][kRound];
    i32x4 x[kRound][W4 ? 2 : 1];
  };
  auto load = [&](int u0, Round& r) {
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
#pragma unroll
      for (int t = 0; t < kSets; ++t)
#pragma unroll
        for (int i = 0; i < TILES; ++i) r.w[t][i][u] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < (W4 ? 2 : 1); ++h) r.x[u][h] = i32x4{0, 0, 0, 0};
      if (u0 + u >= u_end) continue;
      const int byte = (u0 + u) * kUnit;  // activation byte of the unit
      if constexpr (W4) {
        // K is a multiple of 16: each 16-code half is wholly in or out.
        const bool lo = byte + ch * 32 + 16 <= kbytes, hi = byte + ch * 32 + 32 <= kbytes;
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        if (lo) {
#pragma unroll
          for (int t = 0; t < kSets; ++t)
#pragma unroll
            for (int i = 0; i < TILES; ++i) {
              const uint8_t* p = wrow[t][i] + (byte >> 7) * unit_stride;  // byte / 2 in the row layout
              if (hi) {
                r.w[t][i][u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
              } else {
                const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
                r.w[t][i][u] = i32x4{static_cast<int>(v.x), static_cast<int>(v.y), 0, 0};
              }
            }
          r.x[u][0] = *reinterpret_cast<const i32x4*>(xrow + byte);
        }
        if (hi) r.x[u][1] = *reinterpret_cast<const i32x4*>(xrow + byte + 16);
      } else if (byte + ch * 16 < kbytes) {
#pragma unroll
        for (int t = 0; t < kSets; ++t)
#pragma unroll
          for (int i = 0; i < TILES; ++i)
            r.w[t][i][u] =
                __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow[t][i] + (byte >> 6) * unit_stride));
        r.x[u][0] = xload(byte);
      }
    }
  };
  auto mma = [&](const Round& r) {
#pragma unroll
    for (int u = 0; u < kRound; ++u)
#pragma unroll
      for (int t = 0; t < kSets; ++t)
#pragma unroll
        for (int i = 0; i < TILES; ++i) {
          const i32x4 w = r.w[t][i][u];
          if constexpr (W4) {
            acc[t][i] = Mma<I8>::run(expand_w4(w.x, w.y), r.x[u][0], acc[t][i]);
            acc[t][i] = Mma<I8>::run(expand_w4(w.z, w.w), r.x[u][1], acc[t][i]);
          } else {
            acc[t][i] = Mma<I8>::run(w, r.x[u][0], acc[t][i]);
          }
        }
  };
  if constexpr (kDma) {
    // Weights through LDS in whole lines.  A round is two K units: one
    // 128-byte line of each of the 16 rows of every (set, tile) (two int8
    // steps, or 256 int4 codes), fetched by two transfers of 8 rows x 128
    // bytes (lane l: row l / 8 of the half, 16-byte chunk (l % 8) ^ (row % 8)
    // of the line, so that the fragment reads below spread over the LDS
    // banks).  Rounds are double-buffered in the wave's own LDS ring.  Every
    // round issues the same number of transfers and activation loads
    // (addresses clamped into the rows), so a fixed vmcnt retires exactly
    // the previous round; chunks past K or past the wave's range meet zero
    // activations (int4: K % 32 == 0, so a chunk is wholly in or out).
    constexpr int kSlots = kSets * TILES;
    constexpr int kXH = W4 ? 2 : 1;                    // activation loads per unit
    constexpr int kOpsPerRound = 2 * kSlots + (XP ? 0 : 2 * kXH);  // transfers + global activation loads
    const int wbytes = W4 ? kbytes / 2 : kbytes;        // weight bytes of a row
    uint8_t* ring = &wring[wid][0][0][0];
    const int drow = lane >> 3;
    const int dchunk = (lane & 7) ^ drow;
    const uint8_t* dbase[kSets][TILES][2];
#pragma unroll
    for (int t = 0; t < kSets; ++t)
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t nt = n0 + 16 * i;
          const int64_t r = min(nt + 8 * h + drow, static_cast<int64_t>(N) - 1) - nt;
          const int64_t tb = tiled ? (nt & ~int64_t{15}) : nt;
          const int64_t rr = tiled ? (nt & 15) + r : r;
          dbase[t][i][h] = (t == 0 ? B + tb * ldb + rr * pitch1 : epi.B2 + nt * epi.ldb2 + r * pitch2);
        }
    auto issue_w = [&](int u0, int buf) {
      const int wb = u0 * 64;  // weight byte of the round's line
      // chunk dchunk of the line: unit u0 + dchunk / 4, 16-byte piece dchunk % 4
      const int off = wb + dchunk * 16 + 16 <= wbytes ? (u0 + (dchunk >> 2)) * unit_stride + (dchunk & 3) * 16 : 0;
#pragma unroll
      for (int t = 0; t < kSets; ++t)
#pragma unroll
        for (int i = 0; i < TILES; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            gemv_dma16(dbase[t][i][h] + off, ring + (buf * kSlots + t * TILES + i) * 2048 + h * 1024);
    };
    auto issue_x = [&](int u0, i32x4 (&x)[2][kXH], bool (&xv)[2][kXH]) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int hh = 0; hh < kXH; ++hh) {
          const int b = (u0 + q) * kUnit + 16 * hh;  // from this lane's activation base
          xv[q][hh] = u0 + q < u_end && (u0 + q) * kUnit + ch * 16 * kXH + 16 * (hh + 1) <= kbytes;
          x[q][hh] = xload(xv[q][hh] ? b : 0);
        }
    };
    auto issue = [&](int u0, int buf, i32x4 (&x)[2][kXH], bool (&xv)[2][kXH]) {
      issue_w(u0, buf);
      issue_x(u0, x, xv);
    };
    auto consume = [&](int buf, const i32x4 (&x)[2][kXH], const bool (&xv)[2][kXH]) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int off = row * 128 + (((4 * q + ch) ^ (row & 7)) << 4);
        i32x4 xq[kXH];
#pragma unroll
        for (int hh = 0; hh < kXH; ++hh) xq[hh] = xv[q][hh] ? x[q][hh] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < kSets; ++t)
#pragma unroll
          for (int i = 0; i < TILES; ++i) {
            const i32x4 w = *reinterpret_cast<const i32x4*>(ring + (buf * kSlots + t * TILES + i) * 2048 + off);
            if constexpr (W4) {
              acc[t][i] = Mma<I8>::run(expand_w4(w.x, w.y), xq[0], acc[t][i]);
              acc[t][i] = Mma<I8>::run(expand_w4(w.z, w.w), xq[kXH - 1], acc[t][i]);
            } else {
              acc[t][i] = Mma<I8>::run(w, xq[0], acc[t][i]);
            }
          }
      }
    };
    i32x4 xa[2][kXH], xb[2][kXH];
    bool va[2][kXH], vb[2][kXH];
    if (u_begin < u_end) issue_w(u_begin, 0);
    if constexpr (XP) {
      xp_prologue();
      load_epi_in();
    }
    if (u_begin < u_end) issue_x(u_begin, xa, va);
    int buf = 0;
    for (int u0 = u_begin; u0 < u_end; u0 += 4) {
      const bool more = u0 + 2 < u_end;
      if (more) {
        issue(u0 + 2, buf ^ 1, xb, vb);
        gemv_wait_vm<kOpsPerRound>();
      } else {
        gemv_wait_vm<0>();
      }
      consume(buf, xa, va);
      if (!more) break;
      buf ^= 1;
      const bool more2 = u0 + 4 < u_end;
      if (more2) {
        issue(u0 + 4, buf ^ 1, xa, va);
        gemv_wait_vm<kOpsPerRound>();
      } else {
        gemv_wait_vm<0>();
      }
      consume(buf, xb, vb);
      buf ^= 1;
    }
  } else {
  Round ra, rb;
  bool rb_ready = false;
  if constexpr (XP) {
    // Both rounds of weights (up to 2 kRound units per wave) are requested
    // before the prologue packs the activation rows, so that they stream in
    // meanwhile; the activation fragments follow from LDS.
    auto load_w = [&](int u0, Round& r) {
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        const int byte = (u0 + u) * kUnit;
        const bool ok = u0 + u < u_end && byte + ch * 16 < kbytes;
#pragma unroll
        for (int t = 0; t < kSets; ++t)
#pragma unroll
          for (int i = 0; i < TILES; ++i)
            r.w[t][i][u] = ok ? __builtin_nontemporal_load(
                                    reinterpret_cast<const i32x4*>(wrow[t][i] + (byte >> 6) * unit_stride))
                              : i32x4{0, 0, 0, 0};
      }
    };
    auto load_x = [&](int u0, Round& r) {
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        const int byte = (u0 + u) * kUnit;
        r.x[u][0] = u0 + u < u_end && byte + ch * 16 < kbytes ? xload(byte) : i32x4{0, 0, 0, 0};
      }
    };
    if (u_begin < u_end) load_w(u_begin, ra);
    rb_ready = u_begin + kRound < u_end;
    if (rb_ready) load_w(u_begin + kRound, rb);
    xp_prologue();
    load_epi_in();
    if (u_begin < u_end) load_x(u_begin, ra);
    if (rb_ready) load_x(u_begin + kRound, rb);
  } else {
    if (u_begin < u_end) load(u_begin, ra);
  }
  for (int u0 = u_begin; u0 < u_end; u0 += 2 * kRound) {
    if (!rb_ready && u0 + kRound < u_end) load(u0 + kRound, rb);
    rb_ready = false;
    mma(ra);
    if (u0 + kRound >= u_end) break;
    if (u0 + 2 * kRound < u_end) load(u0 + 2 * kRound, ra);
    mma(rb);
  }
  }

  if (WAVES > 1) {
    if (wid > 0) {
#pragma unroll
      for (int t = 0; t < kSets; ++t)
#pragma unroll
        for (int i = 0; i < TILES; ++i) partial[t * TILES + i][wid - 1][lane] = acc[t][i];
    }
    __syncthreads();
    if (wid != 0) return;
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
      for (int t = 0; t < kSets; ++t)
#pragma unroll
        for (int i = 0; i < TILES; ++i) acc[t][i] += partial[t * TILES + i][w][lane];
  }

  if constexpr (SPLIT) {
    // This K range's sums, for the combining launch.
    i32x4* mine = sp.part + ((static_cast<int64_t>(blockIdx.x) * sp.splits + blockIdx.y) * kSets) * 64;
#pragma unroll
    for (int t = 0; t < kSets; ++t) mine[t * 64 + lane] = __builtin_bit_cast(i32x4, acc[t][0]);
  } else {
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      Acc tile[kSets];
#pragma unroll
      for (int t = 0; t < kSets; ++t) tile[t] = acc[t][i];
      tile_epilogue<I8, OUT, ACT, GATED>(tile, lane, n0 + 16 * i, epi_in[i], M, N, C, ldc);
    }
  }
}

// Second launch of the split path: one wave per tile adds the tile's
// partials in K order, then applies the epilogue.
template <bool I8, int OUT, int ACT, bool GATED>
__global__ __launch_bounds__(64) void gemv_combine_kernel(EpiArgs epi, int M, int N, void* __restrict__ C,
                                                          int64_t ldc, SplitArgs sp) {
  using Acc = typename Mma<I8>::Acc;
  constexpr int kSets = GATED ? 2 : 1;
  const int lane = threadIdx.x;
  const i32x4* all = sp.part + static_cast<int64_t>(blockIdx.x) * sp.splits * kSets * 64;
  const EpiIn<GATED> in = load_epi<I8, OUT, GATED>(lane, static_cast<int>(blockIdx.x) * 16, epi, M, N);
  Acc acc[kSets];
#pragma unroll
  for (int t = 0; t < kSets; ++t) {
    Acc sum = __builtin_bit_cast(Acc, all[t * 64 + lane]);
    for (int q = 1; q < sp.splits; ++q) sum += __builtin_bit_cast(Acc, all[(q * kSets + t) * 64 + lane]);
    acc[t] = sum;
  }
  tile_epilogue<I8, OUT, ACT, GATED>(acc, lane, static_cast<int>(blockIdx.x) * 16, in, M, N, C, ldc);
}

inline int gemv_num_cus() { return device_cus(); }

template <bool I8, int OUT, int ACT, bool GATED, bool SPLIT, bool W4, int TILES = 1, bool DMA = false>
void launch_waves(int waves, dim3 grid, const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb,
                  const EpiArgs& epi, int m, int n, int kb, int per, void* C, int64_t ldc, const SplitArgs& sp,
                  bool tiled, bool xtiled, hipStream_t stream) {
  switch (waves) {
    case 4:
      hipLaunchKernelGGL((gemv_kernel<I8, OUT, 4, ACT, GATED, SPLIT, W4, TILES, DMA>), grid, dim3(256), 0, stream, a,
                         lda, b, ldb, epi, m, n, kb, per, C, ldc, sp, tiled, xtiled, XPackArgs{});
      break;
    default:
      hipLaunchKernelGGL((gemv_kernel<I8, OUT, 8, ACT, GATED, SPLIT, W4, TILES, DMA>), grid, dim3(512), 0, stream, a,
                         lda, b, ldb, epi, m, n, kb, per, C, ldc, sp, tiled, xtiled, XPackArgs{});
      break;
  }
}

// Waves per workgroup for `units` K units: four, eight where a wave would
// otherwise stream more than kMaxUnits units (a workgroup's waves split K,
// so fewer waves mean more resident workgroups per CU; a wave's rounds are
// pipelined, so a long range costs no extra latency).
constexpr int kMaxUnits = 32;
inline int waves_for(int64_t units) { return (units + 3) / 4 <= kMaxUnits ? 4 : 8; }

// Few activation rows, few tiles: one workgroup of kWideWaves waves per
// 16-feature tile streams all of K (its waves split K and add through LDS),
// with no split across workgroups and so no combining launch.  For plain
// int8 launches with at most kWideMaxRows rows, fewer tiles than CUs and at
// least two K units per wave.  Measured on the decode down projection
// (1152 x 6912, TILE16 weights), against the split with its combining
// launch: the step 8.7% faster at M = 1, 8% at M = 2, 6% at M = 4, 5% at
// M = 8, 4.5% at M = 12, but 6.6% slower at M = 16, where the sixteen
// activation rows double what each of the few CUs reads.  With the
// activation in the TILE16 layout its fragments are whole lines, and up to
// 16 rows take the wide workgroups (M = 16 step 17.8-17.9 us against
// 18.9-19.1 split, same box).  Each wide workgroup covers 8 features
// (twice the workgroups of 16-feature tiles): down projection at M = 16
// 6.8 against 7.35 us, M = 8 5.85 against 6.45, M = 1 5.2 against 5.1.
constexpr int kWideWaves = 16;
// A wave stages its weights through LDS when it streams at least this many
// K units (a round is two units).
constexpr int kStageMinUnits = 5;
constexpr int64_t kWideMaxRows = 12;
constexpr int64_t kWideMaxRowsTiledX = 16;
bool wide_tiles(int64_t M, int64_t N, int64_t nunits, bool i8, bool w4, int sets, bool xtiled = false) {
  return i8 && !w4 && sets == 1 && M <= (xtiled ? kWideMaxRowsTiledX : kWideMaxRows) &&
         (N + 15) / 16 < gemv_num_cus() && nunits >= 2 * kWideWaves;
}

// How a small-M launch splits K across workgroups: `splits` K ranges of
// `units` K units per 16-feature tile (splits == 1: no split) and the bytes
// of partial sums that needs (kSets x 64 lanes x 16 bytes per tile and
// range).  K is split only when there are fewer tiles than CUs and the
// launch does not take one wide workgroup per tile (the size assumes ROWS
// activations; a TILE16 activation may take the wide workgroups instead and
// leave the workspace unused): aim at two workgroups per CU and keep at
// least 8 MFMA steps per range.
struct SplitPlan {
  int64_t splits;
  int64_t units;
  int64_t bytes;
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t kbytes, int sets, bool w4, bool i8) {
  const int64_t unit = w4 ? 128 : kStepBytes;
  const int64_t nunits = (kbytes + unit - 1) / unit;
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = gemv_num_cus();
  const SplitPlan none{1, nunits, 0};
  if (wide_tiles(M, N, nunits, i8, w4, sets)) return none;
  // int4 weights stream half the bytes per K unit, and the second launch
  // costs more than the split saves (decode down projection, 1152 x 6912,
  // M = 16, same box: 7.4 us unsplit against 8.6 us split with its
  // combining launch; int8: 10.1 against 9.3 us).
  if (w4 || tiles >= cus) return none;
  int64_t splits = std::min<int64_t>((2 * cus + tiles - 1) / tiles, nunits * (unit / kStepBytes) / 8);
  if (splits <= 1) return none;
  const int64_t units = (nunits + splits - 1) / splits;
  splits = (nunits + units - 1) / units;  // no empty range
  if (splits <= 1) return none;
  return SplitPlan{splits, units, tiles * splits * sets * 1024};
}

template <bool I8, int OUT, int ACT = 0, bool GATED = false, bool W4 = false>
hipError_t launch_out(const void* A, int64_t lda, const void* B, int64_t ldb, const EpiArgs& epi, int64_t M,
                      int64_t N, int64_t kbytes, void* C, int64_t ldc, void* ws, hipStream_t stream,
                      bool tiled = false, bool xtiled_in = false) {
  const bool xtiled = xtiled_in && I8 && !W4;  // int8 activations with int8 weights only
  constexpr int kSets = GATED ? 2 : 1;
  constexpr int kUnit = W4 ? 128 : kStepBytes;
  // Weights go through LDS in whole lines when a wave streams enough units
  // for the staging to pay (a round is two units); int4 rows also need
  // K % 32 == 0 so that no 16-byte chunk straddles K.
  constexpr bool kStageable = I8;
  const bool stage_tiled = !(tiled && !W4);
  const bool stage_ok = !W4 || kbytes % 32 == 0;
  const int64_t nunits = (kbytes + kUnit - 1) / kUnit;
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = gemv_num_cus();
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* b = static_cast<const uint8_t*>(B);
  const int m = static_cast<int>(M), n = static_cast<int>(N), kb = static_cast<int>(kbytes);

  // The caller's workspace (validated to hold plan.bytes) enables the split.
  if constexpr (I8 && !W4 && !GATED) {
    if (wide_tiles(M, N, nunits, I8, W4, kSets, xtiled)) {
      const int per = static_cast<int>((nunits + kWideWaves - 1) / kWideWaves);
      const dim3 grid(static_cast<unsigned>((N + 7) / 8));
      const SplitArgs none{nullptr, 1, 0};
      if (per >= kStageMinUnits)
        hipLaunchKernelGGL((gemv_kernel<I8, OUT, kWideWaves, ACT, false, false, false, 1, true>), grid,
                           dim3(64 * kWideWaves), 0, stream, a, lda, b, ldb, epi, m, n, kb, per, C, ldc, none, tiled,
                           xtiled, XPackArgs{});
      else
        hipLaunchKernelGGL((gemv_kernel<I8, OUT, kWideWaves, ACT, false, false, false, 1, false>), grid,
                           dim3(64 * kWideWaves), 0, stream, a, lda, b, ldb, epi, m, n, kb, per, C, ldc, none, tiled,
                           xtiled, XPackArgs{});
      return hipGetLastError();
    }
  }
  const SplitPlan plan = split_plan(M, N, kbytes, kSets, W4, I8);
  if (plan.splits > 1 && ws != nullptr) {
    const int64_t units = plan.units, splits = plan.splits;
    const int waves = waves_for(units);
    const int per = static_cast<int>((units + waves - 1) / waves);
    const SplitArgs sp{reinterpret_cast<i32x4*>(ws), static_cast<int>(splits), static_cast<int>(units)};
    const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(splits));
    if (kStageable && stage_ok && stage_tiled && per >= kStageMinUnits)
      launch_waves<I8, OUT, ACT, GATED, true, W4, 1, kStageable>(waves, grid, a, lda, b, ldb, epi, m, n, kb, per, C,
                                                                 ldc, sp, tiled, xtiled, stream);
    else
      launch_waves<I8, OUT, ACT, GATED, true, W4>(waves, grid, a, lda, b, ldb, epi, m, n, kb, per, C, ldc, sp,
                                                  tiled, xtiled, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_combine_kernel<I8, OUT, ACT, GATED>), dim3(static_cast<unsigned>(tiles)), dim3(64), 0,
                       stream, epi, m, n, C, ldc, sp);
    return hipGetLastError();
  }
  const int waves = waves_for(nunits);
  const int per = static_cast<int>((nunits + waves - 1) / waves);
  // Two tiles per workgroup share every activation fragment once there are
  // at least four tiles per CU (plain launches only; with fewer, the
  // workgroups of two tiles spread unevenly over the CUs).
  const bool stage = kStageable && stage_ok && stage_tiled && per >= kStageMinUnits;
  const SplitArgs none{nullptr, 1, 0};
  if (!GATED && tiles >= 4 * cus) {
    const dim3 grid(static_cast<unsigned>((tiles + 1) / 2));
    if (stage)
      launch_waves<I8, OUT, ACT, GATED, false, W4, GATED ? 1 : 2, kStageable>(waves, grid, a, lda, b, ldb, epi, m, n,
                                                                              kb, per, C, ldc, none, tiled, xtiled, stream);
    else
      launch_waves<I8, OUT, ACT, GATED, false, W4, GATED ? 1 : 2>(waves, grid, a, lda, b, ldb, epi, m, n, kb, per, C,
                                                                  ldc, none, tiled, xtiled, stream);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(tiles));
  if (stage)
    launch_waves<I8, OUT, ACT, GATED, false, W4, 1, kStageable>(waves, grid, a, lda, b, ldb, epi, m, n, kb, per, C,
                                                                ldc, none, tiled, xtiled, stream);
  else
    launch_waves<I8, OUT, ACT, GATED, false, W4>(waves, grid, a, lda, b, ldb, epi, m, n, kb, per, C, ldc, none,
                                                 tiled, xtiled, stream);
  return hipGetLastError();
}

// Launch that packs its own bf16 activation rows (M <= kPackinMaxRows):
// one workgroup per 16-feature tile over all of K, 16 waves for a plain
// linear, 4 for the gated pair (its two weight sets per lane fit four
// waves' registers), one thread per 16-feature chunk of a row in the
// prologue (the caller keeps K <= packin_max_k).  Dynamic LDS: the codes at
// a pitch of K + 16 bytes, four row scales, four rows of wavefront maxima.
template <int OUT, int ACT, bool GATED>
hipError_t launch_out_packin(const XPackArgs& xp, const void* B, int64_t ldb, const EpiArgs& epi, int64_t M,
                             int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t stream, bool tiled) {
  constexpr int kWaves = GATED ? 4 : kWideWaves;
  constexpr int kDynMax = static_cast<int>(kPackinMaxRows) * (16 * 64 * kWaves + 16) + 16 + 16 * kWaves;
  const int64_t nunits = (K + kStepBytes - 1) / kStepBytes;
  const int64_t tiles = (N + 15) / 16;
  const int per = static_cast<int>((nunits + kWaves - 1) / kWaves);
  const int dyn = static_cast<int>(M * (K + 16)) + 16 + 16 * kWaves;
  auto kdma = gemv_kernel<true, OUT, kWaves, ACT, GATED, false, false, 1, true, true>;
  auto kreg = gemv_kernel<true, OUT, kWaves, ACT, GATED, false, false, 1, false, true>;
  // Gated: the register path, where each wave requests its first two rounds
  // of weights before the prologue (the staged path holds one round in LDS;
  // decode gate/up, M = 1: 7.6 against 8.2 us).  Plain: the staged path as
  // in launch_out (its first round issued before the prologue), which
  // measured faster for the 16-wave launch (down projection, M = 1: 8.6
  // against 9.3 us).
  const bool stage = !GATED && per >= kStageMinUnits;
  static std::atomic<uint64_t> lds_dma{0}, lds_reg{0};
  const hipError_t e = stage ? set_lds_limit(reinterpret_cast<const void*>(kdma), kDynMax, lds_dma)
                             : set_lds_limit(reinterpret_cast<const void*>(kreg), kDynMax, lds_reg);
  if (e != hipSuccess) return e;
  const SplitArgs none{nullptr, 1, 0};
  const auto* b = static_cast<const uint8_t*>(B);
  const int m = static_cast<int>(M), n = static_cast<int>(N), kb = static_cast<int>(K);
  if (stage)
    hipLaunchKernelGGL(kdma, dim3(static_cast<unsigned>(tiles)), dim3(64 * kWaves), dyn, stream, nullptr, 0, b, ldb,
                       epi, m, n, kb, per, C, ldc, none, tiled, false, xp);
  else
    hipLaunchKernelGGL(kreg, dim3(static_cast<unsigned>(tiles)), dim3(64 * kWaves), dyn, stream, nullptr, 0, b, ldb,
                       epi, m, n, kb, per, C, ldc, none, tiled, false, xp);
  return hipGetLastError();
}

}  // namespace

int64_t packin_max_k(bool gated) { return 16 * 64 * (gated ? 4 : kWideWaves); }

hipError_t launch_gemv_i8_packin(const void* X, int64_t ldx, int log2g, RotKind kind, const int8_t* signs,
                                 const int8_t* B, int64_t ldb, const float* sb, const float* bias, Act act, int64_t M,
                                 int64_t N, int64_t K, void* C, Elt out, int64_t ldc, hipStream_t stream, bool tiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const XPackArgs xp{X, ldx, log2g, kind == RotKind::Randomized ? 1 : 0, signs};
  const EpiArgs epi{nullptr, sb, bias, nullptr, 0, nullptr, nullptr};
  if (act == Act::None) {
    switch (out) {
      case Elt::F32: return launch_out_packin<0, 0, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled);
      case Elt::BF16: return launch_out_packin<1, 0, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled);
      default: return launch_out_packin<2, 0, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled);
    }
  }
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out_packin<0, 1, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled)
               : launch_out_packin<1, 1, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled);
  return f32 ? launch_out_packin<0, 2, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled)
             : launch_out_packin<1, 2, false>(xp, B, ldb, epi, M, N, K, C, ldc, stream, tiled);
}

hipError_t launch_gemv_i8_gated_packin(const void* X, int64_t ldx, int log2g, RotKind kind, const int8_t* signs,
                                       const int8_t* Bg, int64_t ldbg, const float* sbg, const float* biasg,
                                       const int8_t* Bu, int64_t ldbu, const float* sbu, const float* biasu, Act act,
                                       int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                                       hipStream_t stream, bool tiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const XPackArgs xp{X, ldx, log2g, kind == RotKind::Randomized ? 1 : 0, signs};
  const EpiArgs epi{nullptr, sbg, biasg, reinterpret_cast<const uint8_t*>(Bu), ldbu, sbu, biasu};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out_packin<0, 1, true>(xp, Bg, ldbg, epi, M, N, K, C, ldc, stream, tiled)
               : launch_out_packin<1, 1, true>(xp, Bg, ldbg, epi, M, N, K, C, ldc, stream, tiled);
  return f32 ? launch_out_packin<0, 2, true>(xp, Bg, ldbg, epi, M, N, K, C, ldc, stream, tiled)
             : launch_out_packin<1, 2, true>(xp, Bg, ldbg, epi, M, N, K, C, ldc, stream, tiled);
}

int64_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, bool bf16, bool w4, bool gated) {
  if (N <= 0 || K <= 0) return 0;
  return split_plan(M, N, bf16 ? 2 * K : K, gated ? 2 : 1, w4, !bf16).bytes;
}

hipError_t launch_gemv_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, int64_t M, int64_t N, int64_t K, void* C, Elt out,
                          int64_t ldc, void* ws, hipStream_t stream, bool tiled, bool xtiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  switch (out) {
    case Elt::F32: return launch_out<true, 0>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
    case Elt::BF16: return launch_out<true, 1>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
    default: return launch_out<true, 2>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
  }
}

hipError_t launch_gemv_i8_act(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                              const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K, void* C,
                              Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled, bool xtiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out<true, 0, 1>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled)
               : launch_out<true, 1, 1>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
  return f32 ? launch_out<true, 0, 2>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled)
             : launch_out<true, 1, 2>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
}

hipError_t launch_gemv_i8_gated(const int8_t* A, int64_t lda, const int8_t* Bg, int64_t ldbg, const float* sbg,
                                const float* biasg, const int8_t* Bu, int64_t ldbu, const float* sbu,
                                const float* biasu, const float* sa, Act act, int64_t M, int64_t N, int64_t K,
                                void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled, bool xtiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{sa, sbg, biasg, reinterpret_cast<const uint8_t*>(Bu), ldbu, sbu, biasu};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out<true, 0, 1, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled)
               : launch_out<true, 1, 1, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
  return f32 ? launch_out<true, 0, 2, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled)
             : launch_out<true, 1, 2, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled, xtiled);
}

hipError_t launch_gemv_w4(const int8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K, void* C,
                          Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  if (act == Act::None) {
    switch (out) {
      case Elt::F32: return launch_out<true, 0, 0, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled);
      case Elt::BF16: return launch_out<true, 1, 0, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled);
      default: return launch_out<true, 2, 0, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled);
    }
  }
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out<true, 0, 1, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled)
               : launch_out<true, 1, 1, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled);
  return f32 ? launch_out<true, 0, 2, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled)
             : launch_out<true, 1, 2, false, true>(A, lda, B, ldb, epi, M, N, K, C, ldc, ws, stream, tiled);
}

hipError_t launch_gemv_w4_gated(const int8_t* A, int64_t lda, const uint8_t* Bg, int64_t ldbg, const float* sbg,
                                const float* biasg, const uint8_t* Bu, int64_t ldbu, const float* sbu,
                                const float* biasu, const float* sa, Act act, int64_t M, int64_t N, int64_t K,
                                void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{sa, sbg, biasg, Bu, ldbu, sbu, biasu};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_out<true, 0, 1, true, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled)
               : launch_out<true, 1, 1, true, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled);
  return f32 ? launch_out<true, 0, 2, true, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled)
             : launch_out<true, 1, 2, true, true>(A, lda, Bg, ldbg, epi, M, N, K, C, ldc, ws, stream, tiled);
}

hipError_t launch_gemv_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, const float* bias, int64_t M,
                            int64_t N, int64_t K, void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const EpiArgs epi{nullptr, nullptr, bias, nullptr, 0, nullptr, nullptr};
  // Row strides and K in bytes.
  if (out == Elt::F32) return launch_out<false, 0>(A, 2 * lda, B, 2 * ldb, epi, M, N, 2 * K, C, ldc, ws, stream);
  return launch_out<false, 1>(A, 2 * lda, B, 2 * ldb, epi, M, N, 2 * K, C, ldc, ws, stream);
}

}  // namespace convrot
