// Unquantised bf16 linear (routed layers) on the tiled MFMA kernel; the
// kernel itself is in gemm_kernel.h.
#include "gemm_kernel.h"

namespace convrot {

hipError_t launch_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb, const float* bias, int64_t M,
                            int64_t N, int64_t K, void* C, Elt out, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = static_cast<const uint8_t*>(A);
  const auto* b = static_cast<const uint8_t*>(B);
  const EpiArgs epi{nullptr, nullptr, bias, nullptr, 0, nullptr, nullptr};
  // Row strides and K in bytes.
  if (out == Elt::F32) return launch_gemm<false, 0, 0, false>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
  return launch_gemm<false, 1, 0, false>(a, 2 * lda, b, 2 * ldb, epi, M, N, 2 * K, C, ldc, stream);
}

}  // namespace convrot
