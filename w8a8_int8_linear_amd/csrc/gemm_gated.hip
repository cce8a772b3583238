// Gated pair on the tiled int8 MFMA kernel (gemm_kernel.h): two weights
// sharing one packed activation, Y = act(gate) * up.
#include "gemm_kernel.h"

namespace convrot {

hipError_t launch_gemm_i8_gated(const int8_t* A, int64_t lda, const int8_t* Bg, int64_t ldbg, const float* sbg,
                                const float* biasg, const int8_t* Bu, int64_t ldbu, const float* sbu,
                                const float* biasu, const float* sa, Act act, int64_t M, int64_t N, int64_t K,
                                void* C, Elt out, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto* a = reinterpret_cast<const uint8_t*>(A);
  const auto* bg = reinterpret_cast<const uint8_t*>(Bg);
  const EpiArgs epi{sa, sbg, biasg, reinterpret_cast<const uint8_t*>(Bu), ldbu, sbu, biasu};
  const bool f32 = out == Elt::F32;
  if (act == Act::GeluErf)
    return f32 ? launch_gemm<true, 0, 1, true>(a, lda, bg, ldbg, epi, M, N, K, C, ldc, stream)
               : launch_gemm<true, 1, 1, true>(a, lda, bg, ldbg, epi, M, N, K, C, ldc, stream);
  return f32 ? launch_gemm<true, 0, 2, true>(a, lda, bg, ldbg, epi, M, N, K, C, ldc, stream)
             : launch_gemm<true, 1, 2, true>(a, lda, bg, ldbg, epi, M, N, K, C, ldc, stream);
}

}  // namespace convrot
