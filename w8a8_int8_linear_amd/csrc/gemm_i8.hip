// Quantised linear (plain epilogue).  Whole 128-byte K slices run on the
// eight-wave kernel (gemm_pp.h); a K tail runs on the four-wave kernel
// (gemm_kernel.h).  Both give the same result bits.
#include "gemm_kernel.h"
#include "gemm_pp.h"

namespace convrot {

hipError_t launch_gemm_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, int64_t M, int64_t N, int64_t K, void* C, Elt out,
                          int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = reinterpret_cast<const uint8_t*>(A);
  const auto* b = reinterpret_cast<const uint8_t*>(B);
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  if (pp_eligible(K)) {
    switch (out) {
      case Elt::F32: return launch_gemm_pp<true, 0>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
      case Elt::BF16: return launch_gemm_pp<true, 1>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
      default: return launch_gemm_pp<true, 2>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    }
  }
  switch (out) {
    case Elt::F32: return launch_gemm<true, 0, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    case Elt::BF16: return launch_gemm<true, 1, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    default: return launch_gemm<true, 2, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
  }
}

}  // namespace convrot
