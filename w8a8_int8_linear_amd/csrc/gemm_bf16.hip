// Unquantised bf16 linear (routed layers): the eight-wave kernel
// (gemm_pp.h) when 2 K is a multiple of 128 bytes, else the four-wave
// kernel (gemm_kernel.h).
#include "gemm_kernel.h"
#include "gemm_pp.h"

namespace convrot {

hipError_t launch_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, const float* bias, int64_t M,
                            int64_t N, int64_t K, void* C, Elt out, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* b = static_cast<const uint8_t*>(B);
  const EpiArgs epi{nullptr, nullptr, bias, nullptr, 0, nullptr, nullptr};
  // Row strides and K in bytes.
  if (pp_eligible(2 * K)) {
    if (out == Elt::F32) return launch_gemm_pp<false, 0>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
    return launch_gemm_pp<false, 1>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
  }
  if (out == Elt::F32) return launch_gemm<false, 0, 0, false>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
  return launch_gemm<false, 1, 0, false>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
}

}  // namespace convrot
