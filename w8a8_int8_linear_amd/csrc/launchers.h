// Internal launcher declarations shared by the C-ABI layer (api.cpp) and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

enum class Elt : int { F32 = 0, BF16 = 1, I32 = 2 };
enum class RotKind : int { Regular = 0, Randomized = 1 };
// Activation of a fused epilogue (values of convrot_act).
enum class Act : int { None = 0, GeluErf = 1, GeluTanh = 2 };

// Fused group rotation + whole-row absmax + int8 quantisation of `rows` rows
// of X.  When `q` is null the kernel writes the fp32 rotated rows to `xrot`
// instead (checking mode).  t16: the codes in the TILE16 layout (ldq == K,
// K % 64 == 0, q holding whole tiles of 16 rows).  Shapes were validated by
// the caller.
hipError_t launch_pack_rows(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx,
                            int log2G, RotKind kind, const int8_t* signs,
                            int8_t* q, int64_t ldq, float* scale,
                            float* xrot, int64_t ldr, hipStream_t stream, bool t16 = false);

// The same kernel in int4 weight mode: codes clamped to [-7, 7], scale =
// row max / 7, written as nibble pairs (K / 2 bytes per row of q).
hipError_t launch_pack_rows_w4(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                               RotKind kind, const int8_t* signs, uint8_t* q, int64_t ldq, float* scale,
                               hipStream_t stream);

// int4 nibble pairs [rows, ldq bytes] -> int8 codes [rows, ldd].
hipError_t launch_unpack_w4(const uint8_t* q, int64_t ldq, int64_t rows, int64_t K, int8_t* dst, int64_t ldd,
                            hipStream_t stream);

// Tiled matrix-core GEMM, C = A B^T with both operands K-contiguous.
//   int8 mode : A = Qx [M, K] int8, B = Qw [N, K] int8, exact int32
//               accumulation, epilogue acc * sa[m] * sb[n] + bias[n]
//               (or the raw accumulator when out == I32).
//   bf16 mode : A = X [M, K] bf16, B = W [N, K] bf16, fp32 accumulation,
//               epilogue acc + bias[n].
// lda/ldb/ldc in elements.
hipError_t launch_gemm_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                          const float* sa, const float* sb, const float* bias,
                          int64_t M, int64_t N, int64_t K,
                          void* C, Elt out, int64_t ldc, hipStream_t stream);

hipError_t launch_gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                            const float* bias, int64_t M, int64_t N, int64_t K,
                            void* C, Elt out, int64_t ldc, hipStream_t stream);

// int8 mode with a fused activation, Y = act(A sa sb + bias); `act` is
// GeluErf or GeluTanh and `out` F32 or BF16.
hipError_t launch_gemm_i8_act(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                              const float* sa, const float* sb, const float* bias, Act act,
                              int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                              hipStream_t stream);

// launch_gemm_i8_act that also writes, for the next layer's pack, the
// largest magnitude of every G-group (G = 2^log2g, log2g in {2, 4, 6, 8}) of
// each output row (as stored) after the regular rotation R_G:
// rowmax [M, ldm] fp32.  Needs N % 256 == 0, K % 128 == 0, C aligned for
// 4-element stores (ldc % 4 == 0).
hipError_t launch_gemm_i8_act_rowmax(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, const float* sa,
                                     const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K,
                                     void* C, Elt out, int64_t ldc, float* rowmax, int64_t ldm, int log2g,
                                     hipStream_t stream);

// The pack of rows of X whose per-group maxima of the rotated values are
// given (pmax [rows, ldp], as launch_gemm_i8_act_rowmax writes them): int8
// codes and scales, regular kind, log2G in {2, 4, 6, 8}.  The same bits as
// launch_pack_rows for maxima computed with the same operations.
hipError_t launch_pack_rows_prescaled(const void* X, Elt xdt, int64_t rows, int64_t K, int64_t ldx, int log2G,
                                      const float* pmax, int64_t ldp, int8_t* q, int64_t ldq, float* scale,
                                      hipStream_t stream);

// Gated pair sharing the packed activation A:
//   Y = act(A Bg^T sa sbg + biasg) * (A Bu^T sa sbu + biasu)
// `act` is GeluErf or GeluTanh and `out` F32 or BF16.
hipError_t launch_gemm_i8_gated(const int8_t* A, int64_t lda, const int8_t* Bg, int64_t ldbg,
                                const float* sbg, const float* biasg, const int8_t* Bu, int64_t ldbu,
                                const float* sbu, const float* biasu, const float* sa, Act act,
                                int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                                hipStream_t stream);

// Weight-streaming kernels for small M (M <= kGemvMaxRows).  The int8 one
// gives the same result bits as launch_gemm_i8; the bf16 one computes the
// same as launch_gemm_bf16 up to fp32 summation order.  `ws` is NULL (no
// split over K) or a 16-byte aligned buffer of at least
// gemv_workspace_bytes(...) bytes for the split's partial sums.
constexpr int64_t kGemvMaxRows = 16;
// Partial-sum bytes a small-M launch over M rows, N outputs and K inputs
// splits into on the current device (0: that shape does not split).  bf16:
// the unquantised mode; w4: int4 weights; gated: two weights per launch.
int64_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, bool bf16, bool w4, bool gated);
hipError_t launch_gemv_i8(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                          const float* sa, const float* sb, const float* bias,
                          int64_t M, int64_t N, int64_t K,
                          void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled = false,
                          bool xtiled = false);

// Small-M linears that pack their own activation rows: bf16 X [M, ldx
// elements], M <= kPackinMaxRows, K <= packin_max_k(gated), rotated with
// G = 2^log2g of `kind` and quantised exactly as launch_pack_rows does, then
// the same products and epilogue as launch_gemv_i8 / _i8_gated on those
// codes (the same result bits as packing first).
constexpr int64_t kPackinMaxRows = 4;
int64_t packin_max_k(bool gated);
hipError_t launch_gemv_i8_packin(const void* X, int64_t ldx, int log2g, RotKind kind, const int8_t* signs,
                                 const int8_t* B, int64_t ldb, const float* sb, const float* bias, Act act, int64_t M,
                                 int64_t N, int64_t K, void* C, Elt out, int64_t ldc, hipStream_t stream, bool tiled);
hipError_t launch_gemv_i8_gated_packin(const void* X, int64_t ldx, int log2g, RotKind kind, const int8_t* signs,
                                       const int8_t* Bg, int64_t ldbg, const float* sbg, const float* biasg,
                                       const int8_t* Bu, int64_t ldbu, const float* sbu, const float* biasu, Act act,
                                       int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                                       hipStream_t stream, bool tiled);

hipError_t launch_gemv_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                            const float* bias, int64_t M, int64_t N, int64_t K,
                            void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream);
hipError_t launch_gemv_i8_act(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                              const float* sa, const float* sb, const float* bias, Act act,
                              int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                              void* ws, hipStream_t stream, bool tiled = false, bool xtiled = false);
hipError_t launch_gemv_i8_gated(const int8_t* A, int64_t lda, const int8_t* Bg, int64_t ldbg,
                                const float* sbg, const float* biasg, const int8_t* Bu, int64_t ldbu,
                                const float* sbu, const float* biasu, const float* sa, Act act,
                                int64_t M, int64_t N, int64_t K, void* C, Elt out, int64_t ldc,
                                void* ws, hipStream_t stream, bool tiled = false, bool xtiled = false);

// The weight of a small-M launch in the TILE16 layout (`tiled`): tiles of
// 16 rows, each 64-byte K unit of a tile 1 KiB of consecutive memory; ldb is
// then the bytes of one row.  Needs N % 16 == 0 and whole units.  The int8
// launches above also read the activation A in that layout (`xtiled`: M <=
// 16 rows in one tile, lda == K, K % 64 == 0), whose fragment loads then
// cover whole lines.
//
// TILE16 copy of rows of row_bytes bytes (row_bytes % 64 == 0, rows % 16 ==
// 0): dst receives rows * row_bytes bytes, s_out a copy of s_in [rows].
hipError_t launch_tile_rows(const uint8_t* src, int64_t lds, uint8_t* dst, int64_t rows, int64_t row_bytes,
                            const float* s_in, float* s_out, hipStream_t stream);

// Data-free smoothing of an FFN's intermediate channels (offline): s [F]
// and, where the outputs are non-null, the scaled fp32 weights
// W_up / s (rows) and W_down * s (columns).
hipError_t launch_smooth_ffn(const void* up, Elt up_dt, int64_t ldu, const void* dn, Elt dn_dt, int64_t ldd, int64_t F,
                             int64_t K, int64_t K_out, bool max_norm, float* s, float* up_out, int64_t ldu_out,
                             float* dn_out, int64_t ldd_out, hipStream_t stream);

// Number of K blocks the down product splits K into on the current device
// (1: no split).  With nb > 1 it needs nb * M * r fp32 partials.
int lora_down_blocks(int64_t M, int64_t K, int64_t r);
// T = X A^T rounded to bf16: X bf16 [M, K], A bf16 [r, K] (r % 16 == 0,
// r <= 256), T bf16 [M, ldt]; `partials` (16-byte aligned) holds
// lora_down_blocks(M, K, r) * M * r floats when that count is above 1.
hipError_t launch_lora_down(const void* X, int64_t ldx, const void* A, int64_t lda, int64_t M, int64_t K, int64_t r,
                            void* T, int64_t ldt, float* partials, hipStream_t stream);
// Y[m, n] += scale * sum_j T[m, j] B[n, j]: T bf16 [M, r], B bf16 [N, r]
// (r % 16 == 0, rows 16-byte aligned), Y fp32 or bf16 [M, ldy], in place.
hipError_t launch_lora_up(const void* T, int64_t ldt, const void* B, int64_t ldb, int64_t M, int64_t N, int64_t r,
                          float scale, void* Y, Elt out, int64_t ldy, hipStream_t stream);

// Small-M kernels with int4 weights (nibble pairs, ldb in bytes): the same
// accumulators as the int8 kernels on the expanded codes.  `act` may be
// None (then `out` may be I32) for the plain linear.
hipError_t launch_gemv_w4(const int8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, const float* sa,
                          const float* sb, const float* bias, Act act, int64_t M, int64_t N, int64_t K, void* C,
                          Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled = false);
hipError_t launch_gemv_w4_gated(const int8_t* A, int64_t lda, const uint8_t* Bg, int64_t ldbg, const float* sbg,
                                const float* biasg, const uint8_t* Bu, int64_t ldbu, const float* sbu,
                                const float* biasu, const float* sa, Act act, int64_t M, int64_t N, int64_t K,
                                void* C, Elt out, int64_t ldc, void* ws, hipStream_t stream, bool tiled = false);

}  // namespace convrot
