// Tiled matrix-core GEMM for gfx950: C = A B^T with both operands stored
// K-contiguous ("NT"), fused epilogue.
//
// int8 mode is the quantised linear ("INT8 Convrot Safetensors", section
// "Runtime activation quantization"): A = Qx [M, K], B = Qw [N, K], exact
// int32 accumulation A[r, o] = sum_i Qx[r, i] Qw[o, i], then
// Y[r, o] = A * s_x[r] * s_w[o] + b[o] written as fp32 or bf16 (or the raw
// int32 accumulator).  bf16 mode is the unquantised linear that routed
// layers keep (sglang PR 34581 summary, kitchen_int8 routing): fp32
// accumulation of bf16 products, Y = acc + b.
//
// Design:
//  * 256x256 output tile per 256-thread workgroup, 4 waves in a 2x2 grid,
//    each wave owning a 128x128 sub-tile: 8x8 MFMA tiles of 16x16, i.e. 256
//    int32/fp32 accumulators per lane.  K advances in 128-byte slices.
//  * Both instruction kinds consume 16 bytes per lane per operand and cover
//    64 bytes of K (v_mfma_i32_16x16x64_i8: 64 int8; v_mfma_f32_16x16x32_bf16:
//    32 bf16), so the data movement is shared and only the MFMA differs.
//  * The weight tile feeds the MFMA "row" operand and the activation tile
//    the "column" operand, so each lane's four accumulators are four
//    consecutive output features of one output row (one 16-byte fp32 or
//    8-byte bf16 store).
//  * LDS holds two [256][128 B] slices per operand (128 KiB double buffer).
//    16-byte chunks are XOR-swizzled by (row & 7), which makes both the
//    coalesced row writes and the MFMA fragment reads (16 rows, one chunk
//    column) bank-conflict free.
//  * Slices move global -> LDS directly (global_load_lds_dwordx4, no
//    staging registers); slice k+1 is in flight while the MFMAs of slice k
//    run, with one barrier per slice.
//  * Workgroups are remapped so that each of the 8 XCDs (workgroup id mod 8
//    on dispatch) works on a contiguous range of tiles, and tiles are walked
//    in groups of 8 row-tiles so that concurrent workgroups on one XCD share
//    A and B panels in that XCD's L2.
//  * Integer accumulation is exact, so every tiling gives the same bits.
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;  // bytes of K per LDS slice
constexpr int kWM = 128;
constexpr int kWN = 128;
constexpr int kTM = kWM / 16;
constexpr int kTN = kWN / 16;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kTileBytes = kBM * kBK;            // one operand slice
constexpr int kStageBytes = 2 * kTileBytes;      // A + B slices
constexpr int kSmemBytes = 2 * kStageBytes;      // double buffer
constexpr int kChunksPerThread = kTileBytes / 16 / kThreads;  // per operand

template <bool I8>
struct Mfma;

template <>
struct Mfma<true> {
  typedef i32x4 acc_t;
  static __device__ __forceinline__ i32x4 run(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<false> {
  typedef f32x4 acc_t;
  static __device__ __forceinline__ f32x4 run(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

__device__ __forceinline__ int swizzled(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

// Tile coordinates for this workgroup: XCD-contiguous ranges, then grouped
// row-major order inside each range.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, local = bid / 8;
  const int logical = xcd * q + min(xcd, r) + local;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// OUT: 0 = fp32, 1 = bf16, 2 = raw int32 accumulator.
template <bool I8, int OUT, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    const float* __restrict__ sa, const float* __restrict__ sb, const float* __restrict__ bias, int M, int N,
    int Kb, void* __restrict__ C, int64_t ldc, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  using Op = Mfma<I8>;
  using acc_t = typename Op::acc_t;

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m_blk = tm * kBM;
  const int n_blk = tn * kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = (wid & 1) * kWM;
  const int wn = (wid >> 1) * kWN;

  // Global -> LDS without registers (global_load_lds_dwordx4): one
  // instruction fills a contiguous 1 KiB LDS block, i.e. 8 swizzled rows of
  // the slice, lane l writing physical chunk l % 8 of row l / 8.  Wave w
  // fills blocks w, w + 4, ..., so each lane fetches logical chunk
  // (l % 8) ^ (l / 8) of rows 8 (w + 4 i) + l / 8.  Rows past the matrix edge
  // re-read the last row (their results are never stored).  Offsets are
  // relative to the tile's first row.
  const uint8_t* a_tile = A + static_cast<int64_t>(m_blk) * lda;
  const uint8_t* b_tile = B + static_cast<int64_t>(n_blk) * ldb;
  const int dma_ch = (lane & 7) ^ (lane >> 3);
  int a_off[kChunksPerThread], b_off[kChunksPerThread];
#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) {
    const int row = 8 * (wid + 4 * i) + (lane >> 3);
    a_off[i] = (min(m_blk + row, M - 1) - m_blk) * static_cast<int>(lda) + dma_ch * 16;
    b_off[i] = (min(n_blk + row, N - 1) - n_blk) * static_cast<int>(ldb) + dma_ch * 16;
  }
  auto issue_slice = [&](int buf, int k0) {
    uint8_t* sA = smem + buf * kStageBytes;
    uint8_t* sB = sA + kTileBytes;
    // A chunk past the end of K fetches the row's first chunk instead (a
    // valid address); the tail slice is zero-filled after it lands.
    const int kk = (KTAIL && k0 + dma_ch * 16 >= Kb) ? -dma_ch * 16 : k0;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      __builtin_amdgcn_global_load_lds(a_tile + a_off[i] + kk, (lds_ptr_t)(sA + (wid + 4 * i) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(b_tile + b_off[i] + kk, (lds_ptr_t)(sB + (wid + 4 * i) * 1024), 16, 0, 0);
    }
  };
  auto zero_tail = [&](int buf, int k0) {
    uint8_t* sA = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 3, ch = idx & 7;
      if (k0 + ch * 16 >= Kb) {
        *reinterpret_cast<i32x4*>(sA + swizzled(row, ch)) = i32x4{0, 0, 0, 0};
        *reinterpret_cast<i32x4*>(sA + kTileBytes + swizzled(row, ch)) = i32x4{0, 0, 0, 0};
      }
    }
  };

  acc_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // Fragment addresses: row (l & 15) of each 16-row tile, chunk (l >> 4) of
  // each 64-byte K step; the swizzle term depends on the lane only.
  const int frag_row = lane & 15;
  const int frag_ch = lane >> 4;
  int frag_off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) frag_off[ks] = frag_row * kBK + (((4 * ks + frag_ch) ^ (frag_row & 7)) << 4);

  const int nk = (Kb + kBK - 1) / kBK;
  issue_slice(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue_slice(cur ^ 1, (kt + 1) * kBK);
    if (KTAIL && kt == nk - 1) {
      zero_tail(cur, kt * kBK);
      __syncthreads();
    }
    const uint8_t* sA = smem + cur * kStageBytes;
    const uint8_t* sB = sA + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 fa[kTM], fb[kTN];
#pragma unroll
      for (int i = 0; i < kTM; ++i)
        fa[i] = *reinterpret_cast<const i32x4*>(sA + (wm + 16 * i) * kBK + frag_off[ks]);
#pragma unroll
      for (int j = 0; j < kTN; ++j)
        fb[j] = *reinterpret_cast<const i32x4*>(sB + (wn + 16 * j) * kBK + frag_off[ks]);
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = Op::run(fb[j], fa[i], acc[i][j]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // Epilogue.  Lane holds, for tile (i, j), output row m = m0 + 16 i + (l & 15)
  // and the four consecutive output features n = n0 + 16 j + 4 (l >> 4) + r.
  const int n_lane = 4 * (lane >> 4);
  float s_row[kTM];
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    const int m = min(m_blk + wm + 16 * i + frag_row, M - 1);
    s_row[i] = (I8 && OUT != 2) ? sa[m] : 1.f;
  }
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int n = n_blk + wn + 16 * j + n_lane;
    if (n >= N) continue;
    float s_col[4], b_col[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      s_col[r] = (I8 && OUT != 2) ? sb[nn] : 1.f;
      b_col[r] = (bias && OUT != 2) ? bias[nn] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int m = m_blk + wm + 16 * i + frag_row;
      if (m >= M) continue;
      const acc_t a = acc[i][j];
      if constexpr (OUT == 2) {
        int32_t* out = static_cast<int32_t*>(C) + static_cast<int64_t>(m) * ldc + n;
        if (n + 3 < N && vec_ok(out)) {
          *reinterpret_cast<i32x4*>(out) = a;
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) out[r] = a[r];
        }
      } else {
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (I8) {
            y[r] = fmaf(static_cast<float>(a[r]), s_row[i] * s_col[r], b_col[r]);
          } else {
            y[r] = a[r] + b_col[r];
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
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          __bf16* out = static_cast<__bf16*>(C) + static_cast<int64_t>(m) * ldc + n;
          if (n + 3 < N && vec_ok(out)) {
            *reinterpret_cast<bf16x4*>(out) =
                bf16x4{static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1]), static_cast<__bf16>(y[2]),
                       static_cast<__bf16>(y[3])};
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) out[r] = static_cast<__bf16>(y[r]);
          }
        }
      }
    }
  }
}

template <bool I8, int OUT, bool KTAIL>
hipError_t launch_typed(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const float* sa,
                        const float* sb, const float* bias, int64_t M, int64_t N, int64_t Kb, void* C,
                        int64_t ldc, hipStream_t stream) {
  auto kern = gemm_nt_kernel<I8, OUT, KTAIL>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), kSmemBytes, stream, A, lda, B, ldb, sa, sb, bias,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(Kb), C, ldc, tiles_m, tiles_n);
  return hipGetLastError();
}

template <bool I8, int OUT>
hipError_t launch_ktail(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const float* sa,
                        const float* sb, const float* bias, int64_t M, int64_t N, int64_t Kb, void* C,
                        int64_t ldc, hipStream_t stream) {
  if (Kb % kBK == 0) return launch_typed<I8, OUT, false>(A, lda, B, ldb, sa, sb, bias, M, N, Kb, C, ldc, stream);
  return launch_typed<I8, OUT, true>(A, lda, B, ldb, sa, sb, bias, M, N, Kb, C, ldc, stream);
}

}  // namespace

hipError_t launch_gemm_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, int64_t M, int64_t N, int64_t K, void* C, Elt out,
                          int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint8_t* a = reinterpret_cast<const uint8_t*>(A);
  const uint8_t* b = reinterpret_cast<const uint8_t*>(B);
  switch (out) {
    case Elt::F32: return launch_ktail<true, 0>(a, lda, b, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
    case Elt::BF16: return launch_ktail<true, 1>(a, lda, b, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
    default: return launch_ktail<true, 2>(a, lda, b, ldb, sa, sb, bias, M, N, K, C, ldc, stream);
  }
}

hipError_t launch_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, const float* bias, int64_t M,
                            int64_t N, int64_t K, void* C, Elt out, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const uint8_t* a = static_cast<const uint8_t*>(A);
  const uint8_t* b = static_cast<const uint8_t*>(B);
  if (out == Elt::F32)
    return launch_ktail<false, 0>(a, 2 * lda, b, 2 * ldb, nullptr, nullptr, bias, M, N, 2 * K, C, ldc, stream);
  return launch_ktail<false, 1>(a, 2 * lda, b, 2 * ldb, nullptr, nullptr, bias, M, N, 2 * K, C, ldc, stream);
}

}  // namespace convrot
