// Quantised linear with an activation fused into the epilogue: the
// eight-wave kernel (gemm_pp.h) for whole 128-byte K slices, the four-wave
// kernel (gemm_kernel.h) for a K tail.
#include "gemm_kernel.h"
#include "gemm_pp.h"

namespace convrot {

hipError_t launch_gemm_i8_act(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                              const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K, void* C,
                              Elt out, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = reinterpret_cast<const uint8_t*>(A);
  const auto* b = reinterpret_cast<const uint8_t*>(B);
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  const bool f32 = out == Elt::F32;
  if (pp_eligible(K)) {
    if (act == Act::GeluErf)
      return f32 ? launch_gemm_pp<true, 0, 1>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream)
                 : launch_gemm_pp<true, 1, 1>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    return f32 ? launch_gemm_pp<true, 0, 2>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream)
               : launch_gemm_pp<true, 1, 2>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
  }
  if (act == Act::GeluErf)
    return f32 ? launch_gemm<true, 0, 1, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream)
               : launch_gemm<true, 1, 1, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
  return f32 ? launch_gemm<true, 0, 2, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream)
             : launch_gemm<true, 1, 2, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
}

hipError_t launch_gemm_i8_act_rowmax(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                                     const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K,
                                     void* C, Elt out, int64_t ldc, float* rowmax, int64_t ldm, int log2g,
                                     hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = reinterpret_cast<const uint8_t*>(A);
  const auto* b = reinterpret_cast<const uint8_t*>(B);
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  const RowmaxArgs rm{rowmax, ldm, log2g};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_gemm_pp_rowmax<0, 1>(a, lda, b, ldb, epi, M, N, K, C, ldc, rm, stream)
               : launch_gemm_pp_rowmax<1, 1>(a, lda, b, ldb, epi, M, N, K, C, ldc, rm, stream);
  return f32 ? launch_gemm_pp_rowmax<0, 2>(a, lda, b, ldb, epi, M, N, K, C, ldc, rm, stream)
             : launch_gemm_pp_rowmax<1, 2>(a, lda, b, ldb, epi, M, N, K, C, ldc, rm, stream);
}

}  // namespace convrot
