// Quantised linear on the tiled int8 MFMA kernel (plain epilogue); the
// kernel itself is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace convrot {

hipError_t launch_gemm_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, int64_t M, int64_t N, int64_t K, void* C, Elt out,
                          int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = reinterpret_cast<const uint8_t*>(A);
  const auto* b = reinterpret_cast<const uint8_t*>(B);
  const EpiArgs epi{sa, sb, bias, nullptr, 0, nullptr, nullptr};
  switch (out) {
    case Elt::F32: return launch_gemm<true, 0, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    case Elt::BF16: return launch_gemm<true, 1, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
    default: return launch_gemm<true, 2, 0, false>(a, lda, b, ldb, epi, M, N, K, C, ldc, stream);
  }
}

}  // namespace convrot
