// Runtime LoRA correction added to a linear's output, for gfx950.
//
// "INT8 Convrot Safetensors", LoRA paragraph: adapters are applied at run
// time without touching the int8 weights; the correction is computed from
// the original, unrotated activation and added to the base output.  With the
// adapter's down and up matrices A [r, K] and B [N, r]:
//   T = X A^T              rank-r intermediate, fp32 accumulation, held in
//                          bf16 (the bf16 linear kernels of this library)
//   Y[m, n] += scale * sum_j T[m, j] B[n, j]
// Both products are here, each bound by one operand's bytes:
//  * down (T = X A^T, r <= 256): a workgroup takes up to 64 rows of X, all r
//    columns and one block of K; each wave multiplies its row tiles by every
//    fragment of A it loads (v_mfma_f32_16x16x32_bf16, A's rows as the row
//    operand, from L2), its eight waves split the block and add their partial
//    sums through LDS.  Every workgroup reads A's columns of its block, so the
//    row blocks are made large (A read fewer times) and K is split over
//    workgroups until the grid covers the CUs; the fp32 partials of the K
//    blocks are then added in block order by a small reduction.  T is rounded
//    to bf16 once;
//  * up (Y += scale T B^T): K = r is small, so a launch is bound by reading
//    and writing Y.  A workgroup owns a 64 x 64 block of Y; each wave takes 16
//    rows and four 16-feature MFMA tiles; the block is staged in LDS so that
//    Y is read and written in 16-byte pieces whose every instruction covers
//    whole 128-byte lines; one fused multiply-add per element (bf16 Y:
//    rounded to nearest even).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "launchers.h"

namespace convrot {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 8 bf16 of row `row` at element k (zeros when k is past r).
__device__ __forceinline__ i32x4 load8(const __bf16* base, int64_t ld, int row, int k, int r) {
  if (k >= r) return i32x4{0, 0, 0, 0};
  return *reinterpret_cast<const i32x4*>(base + static_cast<int64_t>(row) * ld + k);
}

// T = X A^T for 16 MT rows of X per workgroup (r <= kMaxRank, r % 16 == 0)
// and the 32-wide k steps [spb y, spb (y + 1)) of K, y = blockIdx.y: each
// wave multiplies its MT row tiles by every fragment of A it loads, and the
// eight waves split the block's steps.  SPLIT: the block's fp32 sum goes to
// P [gridDim.y][M][r]; otherwise (one block) it is rounded into T.
constexpr int kMaxRank = 256;
constexpr int kDownWaves = 8;

template <int RT, int MT, bool SPLIT>  // 16-feature tiles of r, 16-row tiles of X per wave
__global__ __launch_bounds__(64 * kDownWaves) void lora_down_kernel(const __bf16* __restrict__ X, int64_t ldx,
                                                                    const __bf16* __restrict__ A, int64_t lda,
                                                                    int M, int K, int r, int spb,
                                                                    __bf16* __restrict__ T, int64_t ldt,
                                                                    float* __restrict__ P) {
  __shared__ f32x4 partial[kDownWaves - 1][MT * RT][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int row = lane & 15, ch = lane >> 4;
  const int m0 = blockIdx.x * 16 * MT;
  const int steps = (K + 31) / 32;
  const int b0 = blockIdx.y * spb, b1 = min(steps, b0 + spb);
  const int per = (b1 - b0 + kDownWaves - 1) / kDownWaves;
  const int s0 = b0 + wid * per, s1 = min(b1, s0 + per);
  f32x4 acc[MT][RT] = {};
  // One k step of fragments; the next step's are requested before the
  // current step is multiplied.
  struct Frags {
    i32x4 x[MT];
    i32x4 w[RT];
  };
  auto load = [&](int st, Frags& f) {
    const int k = 32 * st + 8 * ch;
#pragma unroll
    for (int i = 0; i < MT; ++i) f.x[i] = load8(X, ldx, min(m0 + 16 * i + row, M - 1), k, K);
#pragma unroll
    for (int j = 0; j < RT; ++j) f.w[j] = 16 * j < r ? load8(A, lda, 16 * j + row, k, K) : i32x4{0, 0, 0, 0};
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      if (16 * j >= r) break;
#pragma unroll
      for (int i = 0; i < MT; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.w[j]),
                                                            __builtin_bit_cast(bf16x8, f.x[i]), acc[i][j], 0, 0, 0);
    }
  };
  Frags fa, fb;
  if (s0 < s1) load(s0, fa);
  for (int st = s0; st < s1; st += 2) {
    if (st + 1 < s1) load(st + 1, fb);
    mma(fa);
    if (st + 1 >= s1) break;
    if (st + 2 < s1) load(st + 2, fa);
    mma(fb);
  }
  if (wid > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < RT; ++j) partial[wid - 1][i * RT + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wid != 0) return;
  // Lane holds row m0 + 16 i + row and features 16 j + 4 ch + e.
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 16 * i + row;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      if (16 * j >= r) break;
      f32x4 v = acc[i][j];
#pragma unroll
      for (int w = 0; w < kDownWaves - 1; ++w) v += partial[w][i * RT + j][lane];
      if (m < M) {
        if constexpr (SPLIT) {
          *reinterpret_cast<f32x4*>(P + (static_cast<int64_t>(blockIdx.y) * M + m) * r + 16 * j + 4 * ch) = v;
        } else {
          *reinterpret_cast<bf16x4*>(T + static_cast<int64_t>(m) * ldt + 16 * j + 4 * ch) =
              bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                     static_cast<__bf16>(v[3])};
        }
      }
    }
  }
}

// T = bf16 of the sum of the nb K blocks' fp32 partials P [nb][M][r], added
// in block order; one thread per 4 features of a row.
__global__ __launch_bounds__(256) void lora_reduce_kernel(const float* __restrict__ P, int M, int r, int nb,
                                                          __bf16* __restrict__ T, int64_t ldt) {
  const int q = r / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * q) return;
  const int64_t m = i / q;
  const int c = 4 * static_cast<int>(i % q);
  f32x4 v = *reinterpret_cast<const f32x4*>(P + m * r + c);
  for (int b = 1; b < nb; ++b) v += *reinterpret_cast<const f32x4*>(P + (static_cast<int64_t>(b) * M + m) * r + c);
  *reinterpret_cast<bf16x4*>(T + m * ldt + c) = bf16x4{static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                                                        static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
}

template <int OUT>
__global__ __launch_bounds__(256) void lora_up_kernel(const __bf16* __restrict__ T, int64_t ldt,
                                                      const __bf16* __restrict__ Bw, int64_t ldb, int M, int N, int r,
                                                      float scale, void* __restrict__ Y, int64_t ldy) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int row = lane & 15, ch = lane >> 4;
  const int m0 = blockIdx.y * 64 + wid * 16;
  const int n0 = blockIdx.x * 64;
  const int mt = min(m0 + row, M - 1);  // rows past the end re-read the last one; their outputs are dropped
  // The workgroup's 64 B rows of each 32-wide k step are loaded once (one
  // 16-byte piece per thread) into LDS and shared by the four waves.
  constexpr int kBPitch = 40;  // bf16 per staged B row (32 + padding across banks)
  __shared__ __bf16 bstage[64 * kBPitch];
  const int br = threadIdx.x >> 2, bp = 8 * (threadIdx.x & 3);
  const int brow = min(n0 + br, N - 1);
  f32x4 acc[4] = {};
  for (int k0 = 0; k0 < r; k0 += 32) {
    const int k = k0 + 8 * ch;
    const i32x4 t = load8(T, ldt, mt, k, r);
    *reinterpret_cast<i32x4*>(&bstage[br * kBPitch + bp]) = load8(Bw, ldb, brow, k0 + bp, r);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x4 b = *reinterpret_cast<const i32x4*>(&bstage[(16 * j + row) * kBPitch + 8 * ch]);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t), __builtin_bit_cast(bf16x8, b),
                                                       acc[j], 0, 0, 0);
    }
    __syncthreads();  // the next step overwrites the staged rows
  }
  // Lane holds rows 4 ch + e (e = 0..3) of the wave's 16 and feature
  // 16 j + row: stage the workgroup's 64 x 64 block in LDS, then update Y in
  // 16-byte pieces laid out so that every load and store instruction of a
  // wave covers whole 128-byte lines (8 rows of 8 bf16 pieces, or 4 rows of
  // 16 fp32 pieces); all of a thread's pieces are requested before any is
  // written.
  __shared__ float stage[64][64 + 4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) stage[16 * wid + 4 * ch + e][16 * j + row] = acc[j][e];
  __syncthreads();
  using out_t = typename std::conditional<OUT == 0, float, __bf16>::type;
  constexpr int kVec = 16 / static_cast<int>(sizeof(out_t));  // elements per piece
  constexpr int kPer = 64 / kVec;                              // threads per row of the block
  constexpr int kRows = 256 / kPer;                            // rows per pass
  constexpr int kPasses = 64 / kRows;
  typedef out_t vec_t __attribute__((ext_vector_type(kVec)));
  const int pr = threadIdx.x / kPer, pc = (threadIdx.x % kPer) * kVec;
  const int n = n0 + pc;
  vec_t old[kPasses];
  bool full[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int m = blockIdx.y * 64 + p * kRows + pr;
    const out_t* y = static_cast<const out_t*>(Y) + static_cast<int64_t>(min(m, M - 1)) * ldy + n;
    full[p] = m < M && n + kVec <= N && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    if (full[p]) old[p] = *reinterpret_cast<const vec_t*>(y);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int tr = p * kRows + pr;
    const int m = blockIdx.y * 64 + tr;
    if (m >= M) continue;
    out_t* y = static_cast<out_t*>(Y) + static_cast<int64_t>(m) * ldy + n;
    const float* v = &stage[tr][pc];
    if (full[p]) {
      vec_t o = old[p];
#pragma unroll
      for (int e = 0; e < kVec; ++e) o[e] = static_cast<out_t>(fmaf(scale, v[e], static_cast<float>(o[e])));
      *reinterpret_cast<vec_t*>(y) = o;
    } else {
      for (int e = 0; e < kVec && n + e < N; ++e) y[e] = static_cast<out_t>(fmaf(scale, v[e], static_cast<float>(y[e])));
    }
  }
}

}  // namespace

// Row tiles per wave by rank: enough to share A's fragments, few enough to
// keep the accumulators in registers and the LDS partials within 112 KiB.
static int lora_row_tiles(int64_t r) { return r <= 64 ? 4 : r <= 128 ? 2 : 1; }

int lora_down_blocks(int64_t M, int64_t K, int64_t r) {
  // Below 128 rows the product takes a few microseconds and the reduction's
  // launch costs more than the split saves (16 rows, K = 1152: 7.5 us
  // unsplit, 8.2 us split in two).
  if (M < 128 || K <= 0) return 1;
  const int cus = device_cus();
  const int64_t rows = 16 * lora_row_tiles(r);
  const int64_t row_blocks = (M + rows - 1) / rows;
  const int64_t steps = (K + 31) / 32;
  // enough K blocks for one workgroup per CU, each block at least two k
  // steps per wave
  int64_t nb = (cus + row_blocks - 1) / row_blocks;
  nb = std::min<int64_t>(nb, std::max<int64_t>(1, steps / (2 * kDownWaves)));
  nb = std::min<int64_t>(nb, 16);
  // no empty block: as many blocks as the per-block step count needs
  const int64_t spb = (steps + nb - 1) / nb;
  return static_cast<int>((steps + spb - 1) / spb);
}

namespace {
template <int RT, int MT>
void launch_down_typed(const __bf16* x, int64_t ldx, const __bf16* a, int64_t lda, int m, int k, int r, int nb,
                       __bf16* t, int64_t ldt, float* p, hipStream_t stream) {
  const int steps = (k + 31) / 32;
  const int spb = (steps + nb - 1) / nb;
  const dim3 grid(static_cast<unsigned>((m + 16 * MT - 1) / (16 * MT)), static_cast<unsigned>(nb));
  if (nb > 1)
    hipLaunchKernelGGL((lora_down_kernel<RT, MT, true>), grid, dim3(64 * kDownWaves), 0, stream, x, ldx, a, lda, m,
                       k, r, spb, t, ldt, p);
  else
    hipLaunchKernelGGL((lora_down_kernel<RT, MT, false>), grid, dim3(64 * kDownWaves), 0, stream, x, ldx, a, lda, m,
                       k, r, spb, t, ldt, p);
}

// mt row tiles per wave, at most MTMAX (a power of two).
template <int RT, int MTMAX>
void launch_down_rt(int mt, const __bf16* x, int64_t ldx, const __bf16* a, int64_t lda, int m, int k, int r, int nb,
                    __bf16* t, int64_t ldt, float* p, hipStream_t stream) {
  if (MTMAX >= 4 && mt >= 4)
    launch_down_typed<RT, (MTMAX >= 4 ? 4 : 1)>(x, ldx, a, lda, m, k, r, nb, t, ldt, p, stream);
  else if (MTMAX >= 2 && mt >= 2)
    launch_down_typed<RT, (MTMAX >= 2 ? 2 : 1)>(x, ldx, a, lda, m, k, r, nb, t, ldt, p, stream);
  else
    launch_down_typed<RT, 1>(x, ldx, a, lda, m, k, r, nb, t, ldt, p, stream);
}
}  // namespace

hipError_t launch_lora_down(const void* X, int64_t ldx, const void* A, int64_t lda, int64_t M, int64_t K, int64_t r,
                            void* T, int64_t ldt, float* partials, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const auto* x = static_cast<const __bf16*>(X);
  const auto* a = static_cast<const __bf16*>(A);
  auto* t = static_cast<__bf16*>(T);
  const int m = static_cast<int>(M), k = static_cast<int>(K), rr = static_cast<int>(r);
  const int nb = lora_down_blocks(M, K, r);
  if (nb > 1 && partials == nullptr) return hipErrorInvalidValue;
  // fewer row tiles when M is small, so a workgroup loads no rows twice
  int mt = lora_row_tiles(r);
  while (mt > 1 && 16 * (mt / 2) >= M) mt /= 2;
  static_assert(kMaxRank == 256, "rank dispatch below covers r <= 256");
  if (r <= 32)
    launch_down_rt<2, 4>(mt, x, ldx, a, lda, m, k, rr, nb, t, ldt, partials, stream);
  else if (r <= 64)
    launch_down_rt<4, 4>(mt, x, ldx, a, lda, m, k, rr, nb, t, ldt, partials, stream);
  else if (r <= 128)
    launch_down_rt<8, 2>(mt, x, ldx, a, lda, m, k, rr, nb, t, ldt, partials, stream);
  else
    launch_down_rt<16, 1>(mt, x, ldx, a, lda, m, k, rr, nb, t, ldt, partials, stream);
  if (nb > 1) {
    const int64_t pieces = M * (r / 4);
    hipLaunchKernelGGL(lora_reduce_kernel, dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, stream,
                       partials, m, rr, nb, t, ldt);
  }
  return hipGetLastError();
}

hipError_t launch_lora_up(const void* T, int64_t ldt, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t r,
                          float scale, void* Y, Elt out, int64_t ldy, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((M + 63) / 64));
  const auto* t = static_cast<const __bf16*>(T);
  const auto* b = static_cast<const __bf16*>(B);
  if (out == Elt::F32)
    hipLaunchKernelGGL(lora_up_kernel<0>, grid, dim3(256), 0, stream, t, ldt, b, ldb, static_cast<int>(M),
                       static_cast<int>(N), static_cast<int>(r), scale, Y, ldy);
  else
    hipLaunchKernelGGL(lora_up_kernel<1>, grid, dim3(256), 0, stream, t, ldt, b, ldb, static_cast<int>(M),
                       static_cast<int>(N), static_cast<int>(r), scale, Y, ldy);
  return hipGetLastError();
}

}  // namespace convrot
