// C ABI of the ConvRot W8A8 linear library: host-side validation, dispatch
// to the gfx950 kernels, status codes and the thread-local error string.
// The declarations and the contract of every entry point are in convrot.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "convrot.h"
#include "device.h"
#include "launchers.h"

namespace {

thread_local char g_last_error[512] = "";

convrot_status fail(convrot_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

convrot_status ok() {
  g_last_error[0] = '\0';
  return CONVROT_OK;
}

convrot_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CONVROT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_size(convrot_dtype d) { return d == CONVROT_BF16 ? 2 : 4; }

int log2_exact(int64_t g) {
  if (g <= 0 || (g & (g - 1)) != 0) return -1;
  int l = 0;
  while ((int64_t{1} << l) < g) ++l;
  return l;
}

// |A| <= K * 127^2 must fit in int32.
constexpr int64_t kMaxK = (int64_t{1} << 31) / (127 * 127) - 1;
// The pack kernel keeps a row in at most 1024 threads x 4 chunks x 16 features.
constexpr int64_t kMaxPackK = 1024 * 4 * 16;
// Grid dimensions.
constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;
// The tiled kernels address a 256-row tile with 32-bit byte offsets.
constexpr int64_t kMaxLdBytes = (int64_t{1} << 31) / 256;

convrot_status check_rot(const convrot_rot& rot, int64_t K, int* log2G) {
  const int lg = log2_exact(rot.group);
  if (rot.kind == CONVROT_ROT_REGULAR) {
    if (lg < 2 || lg > 10 || (lg & 1))
      return fail(CONVROT_ERR_GROUP, "regular rotation needs G in {4, 16, 64, 256, 1024}, got %d", rot.group);
    if (rot.signs != nullptr) return fail(CONVROT_ERR_INVALID_ARG, "regular rotation takes no sign vector");
  } else if (rot.kind == CONVROT_ROT_RANDOMIZED) {
    if (lg < 4 || lg > 10)
      return fail(CONVROT_ERR_GROUP, "randomized rotation needs G = 2^m in [16, 1024], got %d", rot.group);
    if (rot.signs == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "randomized rotation needs a sign vector");
    if (!aligned16(rot.signs)) return fail(CONVROT_ERR_ALIGN, "sign vector must be 16-byte aligned");
  } else {
    return fail(CONVROT_ERR_INVALID_ARG, "unknown rotation kind %d", rot.kind);
  }
  if (K % rot.group != 0)
    return fail(CONVROT_ERR_GROUP, "K = %lld is not a multiple of G = %d", static_cast<long long>(K), rot.group);
  *log2G = lg;
  return CONVROT_OK;
}

convrot_status check_k(int64_t K, int64_t limit) {
  if (K <= 0 || K % 16 != 0)
    return fail(CONVROT_ERR_INVALID_ARG, "K = %lld must be a positive multiple of 16", static_cast<long long>(K));
  if (K > limit)
    return fail(CONVROT_ERR_INVALID_ARG, "K = %lld exceeds the supported maximum %lld", static_cast<long long>(K),
                static_cast<long long>(limit));
  return CONVROT_OK;
}

// Inputs are read in 16-byte chunks: base and row pitch must be 16-byte
// multiples.  Outputs of the linear entry points only need element
// alignment (the kernels fall back to narrower stores where needed).
convrot_status check_matrix(const char* name, const void* p, int64_t rows, int64_t cols, int64_t ld, int elt,
                            bool chunked = true) {
  if (rows > 0 && p == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s is NULL", name);
  if (rows < 0 || rows > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "%s: bad row count", name);
  if (ld < cols)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: leading dimension %lld < %lld", name, static_cast<long long>(ld),
                static_cast<long long>(cols));
  if (!chunked) {
    if ((reinterpret_cast<uintptr_t>(p) % elt) != 0)
      return fail(CONVROT_ERR_ALIGN, "%s must be aligned to its element size", name);
    return CONVROT_OK;
  }
  if (!aligned16(p)) return fail(CONVROT_ERR_ALIGN, "%s must be 16-byte aligned", name);
  if ((ld * elt) % 16 != 0)
    return fail(CONVROT_ERR_ALIGN, "%s: leading dimension x element size must be a multiple of 16 bytes", name);
  return CONVROT_OK;
}

// The layout field of a packed weight: ROWS, or TILE16 with whole tiles of
// 16 rows, dense rows (ld == the row's bytes) and whole 64-byte units.
convrot_status check_layout(const char* name, int32_t layout, int64_t rows, int64_t ld, int64_t row_bytes,
                            int64_t unit_codes, int64_t K) {
  if (layout == CONVROT_LAYOUT_ROWS) return CONVROT_OK;
  if (layout != CONVROT_LAYOUT_TILE16)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: unknown layout %d", name, static_cast<int>(layout));
  if (rows % 16 != 0 || ld != row_bytes || K % unit_codes != 0)
    return fail(CONVROT_ERR_INVALID_ARG,
                "%s: the TILE16 layout needs rows %% 16 == 0 (got %lld), ld == %lld bytes (got %lld) and "
                "K %% %lld == 0 (got %lld)",
                name, static_cast<long long>(rows), static_cast<long long>(row_bytes), static_cast<long long>(ld),
                static_cast<long long>(unit_codes), static_cast<long long>(K));
  return CONVROT_OK;
}

// An activation may take the TILE16 layout too, with dense rows and whole
// 64-byte units; its buffer holds whole tiles of 16 rows (the rows past the
// last are padding).  Only the weight-streaming path reads it (M <= 16, int8
// weights).
convrot_status check_act_layout(const char* name, const convrot_packed* p) {
  if (p->layout == CONVROT_LAYOUT_ROWS) return CONVROT_OK;
  if (p->layout != CONVROT_LAYOUT_TILE16)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: unknown layout %d", name, static_cast<int>(p->layout));
  if (p->ld != p->K || p->K % 64 != 0)
    return fail(CONVROT_ERR_INVALID_ARG,
                "%s: a TILE16 activation needs ld == K (got ld %lld, K %lld) and K %% 64 == 0", name,
                static_cast<long long>(p->ld), static_cast<long long>(p->K));
  return CONVROT_OK;
}

convrot_status check_packed(const char* name, const convrot_packed* p, int* log2G, bool activation) {
  if (p == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s descriptor is NULL", name);
  convrot_status st = check_k(p->K, kMaxK);
  if (st != CONVROT_OK) return st;
  st = check_rot(p->rot, p->K, log2G);
  if (st != CONVROT_OK) return st;
  st = check_matrix(name, p->q, p->rows, p->K, p->ld, 1);
  if (st != CONVROT_OK) return st;
  if (p->rows > 0 && p->scale == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s scale is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p->scale) & 3u) != 0)
    return fail(CONVROT_ERR_ALIGN, "%s scale must be 4-byte aligned", name);
  if (activation) return check_act_layout(name, p);
  return check_layout(name, p->layout, p->rows, p->ld, p->K, 64, p->K);
}

convrot_status check_packed(const char* name, const convrot_packed* p, int* log2G) {
  return check_packed(name, p, log2G, false);
}

// Only the weight-streaming path (M <= 16) reads the tiled layout.
convrot_status check_rows_layout(const char* name, int32_t layout) {
  if (layout != CONVROT_LAYOUT_ROWS)
    return fail(CONVROT_ERR_INVALID_ARG, "%s must be in the ROWS layout", name);
  return CONVROT_OK;
}

convrot_status check_weight_layout_for_m(const char* fn, int32_t layout, int64_t M) {
  if (layout == CONVROT_LAYOUT_TILE16 && M > convrot::kGemvMaxRows)
    return fail(CONVROT_ERR_INVALID_ARG,
                "%s: a TILE16 weight serves M <= %d only (M = %lld); use the ROWS layout for larger M", fn,
                convrot::kGemvMaxRows, static_cast<long long>(M));
  return CONVROT_OK;
}

convrot_status pack_impl(const char* what, const void* X, convrot_dtype xdt, int64_t ldx,
                         const convrot_packed* out, void* stream, bool activation) {
  int log2G = 0;
  if (out == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: output descriptor is NULL", what);
  convrot_status st = check_k(out->K, kMaxPackK);
  if (st != CONVROT_OK) return st;
  st = check_packed("packed output", out, &log2G, activation);
  if (st != CONVROT_OK) return st;
  if (!activation) {
    st = check_rows_layout("packed output", out->layout);
    if (st != CONVROT_OK) return st;
  }
  if (xdt != CONVROT_F32 && xdt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "%s: input must be CONVROT_F32 or CONVROT_BF16", what);
  st = check_matrix("input", X, out->rows, out->K, ldx, elt_size(xdt));
  if (st != CONVROT_OK) return st;
  if (out->rows == 0) return ok();
  const hipError_t e = convrot::launch_pack_rows(
      X, static_cast<convrot::Elt>(xdt), out->rows, out->K, ldx, log2G,
      static_cast<convrot::RotKind>(out->rot.kind), out->rot.signs, out->q, out->ld, out->scale, nullptr, 0,
      static_cast<hipStream_t>(stream), out->layout == CONVROT_LAYOUT_TILE16);
  return from_hip(e, what);
}

// Checks shared by the quantised linear entry points: a packed activation
// and a packed weight that belong together, a bias and an output of Y.
convrot_status check_linear(const char* fn, const convrot_packed* act, const convrot_packed* w, const float* bias,
                            const void* Y, convrot_dtype ydt, int64_t ldy, bool i32_ok) {
  int lga = 0, lgw = 0;
  convrot_status st = check_packed("activation", act, &lga, true);
  if (st != CONVROT_OK) return st;
  st = check_packed("weight", w, &lgw);
  if (st != CONVROT_OK) return st;
  if (act->layout == CONVROT_LAYOUT_TILE16 && act->rows > convrot::kGemvMaxRows)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: a TILE16 activation serves M <= %d only (M = %lld)", fn,
                convrot::kGemvMaxRows, static_cast<long long>(act->rows));
  st = check_weight_layout_for_m(fn, w->layout, act->rows);
  if (st != CONVROT_OK) return st;
  if (act->K != w->K)
    return fail(CONVROT_ERR_MISMATCH, "activation K = %lld but weight K = %lld", static_cast<long long>(act->K),
                static_cast<long long>(w->K));
  if (act->rot.group != w->rot.group || act->rot.kind != w->rot.kind || act->rot.signs != w->rot.signs)
    return fail(CONVROT_ERR_MISMATCH,
                "activation and weight were packed with different rotations (G %d/%d, kind %d/%d, signs %p/%p)",
                act->rot.group, w->rot.group, act->rot.kind, w->rot.kind, static_cast<const void*>(act->rot.signs),
                static_cast<const void*>(w->rot.signs));
  if (ydt != CONVROT_F32 && ydt != CONVROT_BF16 && !(i32_ok && ydt == CONVROT_I32))
    return fail(CONVROT_ERR_DTYPE, "%s: output must be CONVROT_F32 or CONVROT_BF16%s", fn,
                i32_ok ? " or CONVROT_I32" : "");
  st = check_matrix("Y", Y, act->rows, w->rows, ldy, elt_size(ydt), false);
  if (st != CONVROT_OK) return st;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)
    return fail(CONVROT_ERR_ALIGN, "bias must be 4-byte aligned");
  if (act->ld > kMaxLdBytes || w->ld > kMaxLdBytes)
    return fail(CONVROT_ERR_INVALID_ARG, "leading dimension of a packed operand exceeds %lld bytes",
                static_cast<long long>(kMaxLdBytes));
  return CONVROT_OK;
}

convrot_status check_packed_w4(const char* name, const convrot_packed_w4* p, int* log2G) {
  if (p == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s descriptor is NULL", name);
  convrot_status st = check_k(p->K, kMaxK);
  if (st != CONVROT_OK) return st;
  st = check_rot(p->rot, p->K, log2G);
  if (st != CONVROT_OK) return st;
  // Nibble rows are read and written in 8-byte units: base 16-byte aligned,
  // row pitch a multiple of 8 bytes (K / 2 always is).
  if (p->rows > 0 && p->q == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s is NULL", name);
  if (p->rows < 0 || p->rows > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "%s: bad row count", name);
  if (p->ld < p->K / 2)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: leading dimension %lld < K / 2 = %lld bytes", name,
                static_cast<long long>(p->ld), static_cast<long long>(p->K / 2));
  if (!aligned16(p->q)) return fail(CONVROT_ERR_ALIGN, "%s must be 16-byte aligned", name);
  if (p->ld % 8 != 0) return fail(CONVROT_ERR_ALIGN, "%s: leading dimension must be a multiple of 8 bytes", name);
  if (p->rows > 0 && p->scale == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s scale is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p->scale) & 3u) != 0)
    return fail(CONVROT_ERR_ALIGN, "%s scale must be 4-byte aligned", name);
  if (p->ld > kMaxLdBytes)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: leading dimension exceeds %lld bytes", name,
                static_cast<long long>(kMaxLdBytes));
  return check_layout(name, p->layout, p->rows, p->ld, p->K / 2, 128, p->K);
}

// An int4 weight seen through the int8 descriptor checks of check_linear:
// the same K, rotation, row count and layout (the code pointer is only
// compared; a tiled view passes the int8 tile checks since K % 128 == 0).
convrot_packed as_int8_view(const convrot_packed_w4& w) {
  return convrot_packed{reinterpret_cast<int8_t*>(w.q), w.scale, w.rows, w.K, w.K, w.rot, w.layout};
}

// M > 16 with int4 weights: the expanded codes go to the caller's workspace.
convrot_status check_workspace(const void* ws, int64_t ws_bytes, int64_t need) {
  if (ws == nullptr || ws_bytes < need)
    return fail(CONVROT_ERR_INVALID_ARG, "this call needs a workspace of %lld bytes (got %lld)",
                static_cast<long long>(need), static_cast<long long>(ws == nullptr ? 0 : ws_bytes));
  if (!aligned16(ws)) return fail(CONVROT_ERR_ALIGN, "workspace must be 16-byte aligned");
  return CONVROT_OK;
}

// Copy of a ROWS weight into the TILE16 layout (row_bytes per row: K for
// int8 codes, K / 2 for int4 nibble pairs).
template <typename D>
convrot_status tile_impl(const char* what, const D* in, const D* out, int64_t row_bytes, void* stream,
                         convrot_status (*check)(const char*, const D*, int*)) {
  int lgi = 0, lgo = 0;
  convrot_status st = check("input", in, &lgi);
  if (st != CONVROT_OK) return st;
  st = check("output", out, &lgo);
  if (st != CONVROT_OK) return st;
  st = check_rows_layout("input", in->layout);
  if (st != CONVROT_OK) return st;
  if (out->layout != CONVROT_LAYOUT_TILE16)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: the output descriptor must have the TILE16 layout", what);
  if (in->rows != out->rows || in->K != out->K || in->rot.group != out->rot.group || in->rot.kind != out->rot.kind ||
      in->rot.signs != out->rot.signs)
    return fail(CONVROT_ERR_MISMATCH, "%s: input and output differ in rows, K or rotation", what);
  if (in->rows == 0) return ok();
  const auto* src = reinterpret_cast<const uint8_t*>(in->q);
  auto* dst = reinterpret_cast<uint8_t*>(out->q);
  if (src < dst + out->rows * row_bytes && dst < src + (in->rows - 1) * in->ld + row_bytes)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: input and output overlap", what);
  return from_hip(convrot::launch_tile_rows(src, in->ld, dst, in->rows, row_bytes, in->scale, out->scale,
                                            static_cast<hipStream_t>(stream)),
                  what);
}

// Optional split-K workspace of a small-M call: NULL selects the unsplit
// kernel; a non-NULL one must hold the split's partial sums.
convrot_status check_split_workspace(const void* ws, int64_t ws_bytes, int64_t need) {
  if (ws == nullptr) return CONVROT_OK;
  if (ws_bytes < need)
    return fail(CONVROT_ERR_INVALID_ARG, "workspace of %lld bytes is smaller than the %lld this call splits K into",
                static_cast<long long>(ws_bytes), static_cast<long long>(need));
  if (!aligned16(ws)) return fail(CONVROT_ERR_ALIGN, "workspace must be 16-byte aligned");
  return CONVROT_OK;
}

// Workspace a small-M (M <= 16) call of `kind` splits K into.
int64_t small_m_workspace(convrot_linear_kind kind, int64_t M, int64_t N, int64_t K) {
  const bool gated = kind == CONVROT_LINEAR_GATED || kind == CONVROT_LINEAR_W4_GATED;
  const bool w4 = kind == CONVROT_LINEAR_W4 || kind == CONVROT_LINEAR_W4_GATED;
  return convrot::gemv_workspace_bytes(M, N, K, kind == CONVROT_LINEAR_BF16, w4, gated);
}

convrot_status check_act(convrot_act fn) {
  if (fn != CONVROT_ACT_GELU_ERF && fn != CONVROT_ACT_GELU_TANH)
    return fail(CONVROT_ERR_INVALID_ARG, "activation must be CONVROT_ACT_GELU_ERF or CONVROT_ACT_GELU_TANH");
  return CONVROT_OK;
}

// Checks of a linear that packs its own activation rows: bf16 X [M, ldx]
// with 16-byte aligned rows, at most kPackinMaxRows rows, a weight whose K
// the launch covers with one 16-feature chunk per thread, and Y [M, N].
convrot_status check_packin(const char* fn, const void* X, convrot_dtype xdt, int64_t ldx, int64_t M,
                            const convrot_packed* w, const float* bias, const void* Y, convrot_dtype ydt, int64_t ldy,
                            bool gated, bool i32_ok, int* log2G) {
  if (w == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: weight descriptor is NULL", fn);
  convrot_status st = check_packed("weight", w, log2G);
  if (st != CONVROT_OK) return st;
  if (xdt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "%s: X must be CONVROT_BF16 (pack other inputs with convrot_pack_act)", fn);
  if (M < 0 || M > convrot::kPackinMaxRows)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: M = %lld; a packing linear takes 0 to %lld rows", fn,
                static_cast<long long>(M), static_cast<long long>(convrot::kPackinMaxRows));
  if (w->K > convrot::packin_max_k(gated))
    return fail(CONVROT_ERR_INVALID_ARG, "%s: K = %lld exceeds the %lld a packing launch covers", fn,
                static_cast<long long>(w->K), static_cast<long long>(convrot::packin_max_k(gated)));
  st = check_matrix("X", X, M, w->K, ldx, 2);
  if (st != CONVROT_OK) return st;
  if (ydt != CONVROT_F32 && ydt != CONVROT_BF16 && !(i32_ok && ydt == CONVROT_I32))
    return fail(CONVROT_ERR_DTYPE, "%s: output must be CONVROT_F32 or CONVROT_BF16%s", fn,
                i32_ok ? " or CONVROT_I32" : "");
  st = check_matrix("Y", Y, M, w->rows, ldy, elt_size(ydt), false);
  if (st != CONVROT_OK) return st;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)
    return fail(CONVROT_ERR_ALIGN, "bias must be 4-byte aligned");
  if (w->ld > kMaxLdBytes)
    return fail(CONVROT_ERR_INVALID_ARG, "leading dimension of the packed weight exceeds %lld bytes",
                static_cast<long long>(kMaxLdBytes));
  return CONVROT_OK;
}

}  // namespace

extern "C" {

convrot_status convrot_pack_act(const void* X, convrot_dtype xdt, int64_t ldx, const convrot_packed* out,
                                void* stream) {
  return pack_impl("convrot_pack_act", X, xdt, ldx, out, stream, true);
}

convrot_status convrot_pack_weight(const void* W, convrot_dtype wdt, int64_t ldw, const convrot_packed* out,
                                   void* stream) {
  return pack_impl("convrot_pack_weight", W, wdt, ldw, out, stream, false);
}

convrot_status convrot_linear(const convrot_packed* act, const convrot_packed* w, const float* bias, void* Y,
                              convrot_dtype ydt, int64_t ldy, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  convrot_status st = check_linear("convrot_linear", act, w, bias, Y, ydt, ldy, true);
  if (st != CONVROT_OK) return st;
  const int64_t M = act->rows, N = w->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  const auto out = static_cast<convrot::Elt>(ydt);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_PLAIN, M, N, K));
    if (st != CONVROT_OK) return st;
    e = convrot::launch_gemv_i8(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, M, N, K, Y, out, ldy,
                                workspace, s, w->layout == CONVROT_LAYOUT_TILE16,
                                act->layout == CONVROT_LAYOUT_TILE16);
  } else {
    e = convrot::launch_gemm_i8(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, M, N, K, Y, out, ldy, s);
  }
  return from_hip(e, "convrot_linear");
}

}  // extern "C"

namespace {
// Scratch of convrot_linear_noalloc: file-scope device memory for the
// small-M K split's partial sums.  Every GPU the library runs on holds its
// own copy until the process ends.  On the host `scratch` names a host-side
// stand-in, not a device address: host code only ever uses the address
// hipGetSymbolAddress returns for the current device, resolved once per
// device on that device's first call and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[convrot::kMaxDevices];

convrot_status scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "convrot_linear_noalloc: hipGetDevice");
  if (dev < 0 || dev >= convrot::kMaxDevices)
    return fail(CONVROT_ERR_INVALID_ARG, "convrot_linear_noalloc: device %d beyond the %d supported", dev,
                convrot::kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CONVROT_ERR_HIP, "convrot_linear_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return CONVROT_OK;
}
}  // namespace

extern "C" {

convrot_status convrot_linear_noalloc(const convrot_packed* act, const convrot_packed* w, const float* bias, void* Y,
                                      convrot_dtype ydt, int64_t ldy, void* stream) {
  const char* what = "convrot_linear_noalloc";
  convrot_status st = check_linear(what, act, w, bias, Y, ydt, ldy, true);
  if (st != CONVROT_OK) return st;
  const int64_t M = act->rows, N = w->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  const auto out = static_cast<convrot::Elt>(ydt);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (M <= convrot::kGemvMaxRows) {
    const int64_t need = small_m_workspace(CONVROT_LINEAR_PLAIN, M, N, K);
    if (need > CONVROT_NOALLOC_SCRATCH_BYTES)
      return fail(CONVROT_ERR_INVALID_ARG,
                  "%s: this shape splits K into %lld bytes of partial sums, beyond the %d-byte static scratch "
                  "(use convrot_linear with a workspace)",
                  what, static_cast<long long>(need), CONVROT_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
      st = scratch_address(&ws);
      if (st != CONVROT_OK) return st;
    }
    e = convrot::launch_gemv_i8(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, M, N, K, Y, out, ldy, ws,
                                s, w->layout == CONVROT_LAYOUT_TILE16, act->layout == CONVROT_LAYOUT_TILE16);
  } else {
    e = convrot::launch_gemm_i8(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, M, N, K, Y, out, ldy, s);
  }
  return from_hip(e, what);
}

convrot_status convrot_linear_workspace_bytes(convrot_linear_kind kind, int64_t M, int64_t N, int64_t K,
                                              int64_t* bytes) {
  const char* what = "convrot_linear_workspace_bytes";
  if (bytes == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: bytes is NULL", what);
  if (kind < CONVROT_LINEAR_PLAIN || kind > CONVROT_LINEAR_W4_GATED)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: unknown linear kind %d", what, static_cast<int>(kind));
  const convrot_status st = check_k(K, kind == CONVROT_LINEAR_BF16 ? int64_t{1} << 30 : kMaxK);
  if (st != CONVROT_OK) return st;
  if (M < 0 || M > kMaxRows || N < 0 || N > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "%s: bad M or N", what);
  if (M == 0 || N == 0) {
    *bytes = 0;
  } else if (M <= convrot::kGemvMaxRows) {
    *bytes = small_m_workspace(kind, M, N, K);
  } else {
    *bytes = kind == CONVROT_LINEAR_W4 ? N * K : kind == CONVROT_LINEAR_W4_GATED ? 2 * N * K : 0;
  }
  return ok();
}

convrot_status convrot_linear_act(const convrot_packed* act, const convrot_packed* w, const float* bias,
                                  convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  convrot_status st = check_act(fn);
  if (st != CONVROT_OK) return st;
  st = check_linear("convrot_linear_act", act, w, bias, Y, ydt, ldy, false);
  if (st != CONVROT_OK) return st;
  const int64_t M = act->rows, N = w->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_PLAIN, M, N, K));
    if (st != CONVROT_OK) return st;
  }
  const auto out = static_cast<convrot::Elt>(ydt);
  const auto a = static_cast<convrot::Act>(fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      M <= convrot::kGemvMaxRows
          ? convrot::launch_gemv_i8_act(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, a, M, N, K, Y,
                                        out, ldy, workspace, s, w->layout == CONVROT_LAYOUT_TILE16,
                                        act->layout == CONVROT_LAYOUT_TILE16)
          : convrot::launch_gemm_i8_act(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, a, M, N, K, Y,
                                        out, ldy, s);
  return from_hip(e, "convrot_linear_act");
}

convrot_status convrot_linear_act_rowmax(const convrot_packed* act, const convrot_packed* w, const float* bias,
                                         convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, int32_t group_next,
                                         float* rowmax, int64_t ldm, void* stream) {
  const char* what = "convrot_linear_act_rowmax";
  convrot_status st = check_act(fn);
  if (st != CONVROT_OK) return st;
  st = check_linear(what, act, w, bias, Y, ydt, ldy, false);
  if (st != CONVROT_OK) return st;
  st = check_rows_layout("activation", act->layout);
  if (st != CONVROT_OK) return st;
  const int lg = log2_exact(group_next);
  if (lg < 2 || lg > 8 || (lg & 1))
    return fail(CONVROT_ERR_GROUP, "%s: group_next must be 4, 16, 64 or 256, got %d", what, group_next);
  const int64_t M = act->rows, N = w->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  if (M <= convrot::kGemvMaxRows)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: needs M > %lld (the tiled kernel); use convrot_linear_act and "
                "convrot_pack_act", what, static_cast<long long>(convrot::kGemvMaxRows));
  if (N % 256 != 0 || K % 128 != 0)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: needs N %% 256 == 0 and K %% 128 == 0 (N = %lld, K = %lld)", what,
                static_cast<long long>(N), static_cast<long long>(K));
  if (reinterpret_cast<uintptr_t>(Y) % (4 * elt_size(ydt)) != 0 || ldy % 4 != 0)
    return fail(CONVROT_ERR_ALIGN, "%s: Y rows must be aligned for 4-element stores", what);
  st = check_matrix("rowmax", rowmax, M, N / group_next, ldm, 4, false);
  if (st != CONVROT_OK) return st;
  const hipError_t e = convrot::launch_gemm_i8_act_rowmax(
      act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, static_cast<convrot::Act>(fn), M, N, K, Y,
      static_cast<convrot::Elt>(ydt), ldy, rowmax, ldm, lg, static_cast<hipStream_t>(stream));
  return from_hip(e, what);
}

convrot_status convrot_pack_act_rowmax(const void* X, convrot_dtype xdt, int64_t ldx, const float* rowmax,
                                       int64_t ldm, const convrot_packed* out, void* stream) {
  const char* what = "convrot_pack_act_rowmax";
  int log2G = 0;
  if (out == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: output descriptor is NULL", what);
  convrot_status st = check_k(out->K, kMaxPackK);
  if (st != CONVROT_OK) return st;
  st = check_packed("packed output", out, &log2G);
  if (st != CONVROT_OK) return st;
  st = check_rows_layout("packed output", out->layout);
  if (st != CONVROT_OK) return st;
  if (out->rot.kind != CONVROT_ROT_REGULAR || log2G > 8)
    return fail(CONVROT_ERR_GROUP, "%s: given maxima need the regular rotation with G in {4, 16, 64, 256}", what);
  if (xdt != CONVROT_F32 && xdt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "%s: input must be CONVROT_F32 or CONVROT_BF16", what);
  st = check_matrix("input", X, out->rows, out->K, ldx, elt_size(xdt));
  if (st != CONVROT_OK) return st;
  st = check_matrix("rowmax", rowmax, out->rows, out->K >> log2G, ldm, 4, false);
  if (st != CONVROT_OK) return st;
  if (out->rows == 0) return ok();
  const hipError_t e = convrot::launch_pack_rows_prescaled(X, static_cast<convrot::Elt>(xdt), out->rows, out->K, ldx,
                                                           log2G, rowmax, ldm, out->q, out->ld, out->scale,
                                                           static_cast<hipStream_t>(stream));
  return from_hip(e, what);
}

convrot_status convrot_linear_gated(const convrot_packed* act, const convrot_packed* w_gate, const float* b_gate,
                                    const convrot_packed* w_up, const float* b_up, convrot_act fn, void* Y,
                                    convrot_dtype ydt, int64_t ldy, void* workspace, int64_t workspace_bytes,
                                    void* stream) {
  convrot_status st = check_act(fn);
  if (st != CONVROT_OK) return st;
  st = check_linear("convrot_linear_gated", act, w_gate, b_gate, Y, ydt, ldy, false);
  if (st != CONVROT_OK) return st;
  st = check_linear("convrot_linear_gated", act, w_up, b_up, Y, ydt, ldy, false);
  if (st != CONVROT_OK) return st;
  if (w_gate->rows != w_up->rows)
    return fail(CONVROT_ERR_MISMATCH, "gate has %lld output rows but up has %lld",
                static_cast<long long>(w_gate->rows), static_cast<long long>(w_up->rows));
  if (w_gate->layout != w_up->layout)
    return fail(CONVROT_ERR_INVALID_ARG, "convrot_linear_gated: gate and up weights must have the same layout");
  const int64_t M = act->rows, N = w_gate->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_GATED, M, N, K));
    if (st != CONVROT_OK) return st;
  }
  const auto out = static_cast<convrot::Elt>(ydt);
  const auto a = static_cast<convrot::Act>(fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      M <= convrot::kGemvMaxRows
          ? convrot::launch_gemv_i8_gated(act->q, act->ld, w_gate->q, w_gate->ld, w_gate->scale, b_gate, w_up->q,
                                          w_up->ld, w_up->scale, b_up, act->scale, a, M, N, K, Y, out, ldy,
                                          workspace, s, w_gate->layout == CONVROT_LAYOUT_TILE16,
                                          act->layout == CONVROT_LAYOUT_TILE16)
          : convrot::launch_gemm_i8_gated(act->q, act->ld, w_gate->q, w_gate->ld, w_gate->scale, b_gate, w_up->q,
                                          w_up->ld, w_up->scale, b_up, act->scale, a, M, N, K, Y, out, ldy, s);
  return from_hip(e, "convrot_linear_gated");
}

convrot_status convrot_linear_packin(const void* X, convrot_dtype xdt, int64_t ldx, int64_t M, const convrot_packed* w,
                                     const float* bias, convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy,
                                     void* stream) {
  const char* what = "convrot_linear_packin";
  if (fn != CONVROT_ACT_NONE && fn != CONVROT_ACT_GELU_ERF && fn != CONVROT_ACT_GELU_TANH)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: unknown activation %d", what, static_cast<int>(fn));
  int log2G = 0;
  convrot_status st = check_packin(what, X, xdt, ldx, M, w, bias, Y, ydt, ldy, false, fn == CONVROT_ACT_NONE, &log2G);
  if (st != CONVROT_OK) return st;
  if (M == 0 || w->rows == 0) return ok();
  const hipError_t e = convrot::launch_gemv_i8_packin(
      X, ldx, log2G, static_cast<convrot::RotKind>(w->rot.kind), w->rot.signs, w->q, w->ld, w->scale, bias,
      static_cast<convrot::Act>(fn), M, w->rows, w->K, Y, static_cast<convrot::Elt>(ydt), ldy,
      static_cast<hipStream_t>(stream), w->layout == CONVROT_LAYOUT_TILE16);
  return from_hip(e, what);
}

convrot_status convrot_linear_gated_packin(const void* X, convrot_dtype xdt, int64_t ldx, int64_t M,
                                           const convrot_packed* w_gate, const float* b_gate,
                                           const convrot_packed* w_up, const float* b_up, convrot_act fn, void* Y,
                                           convrot_dtype ydt, int64_t ldy, void* stream) {
  const char* what = "convrot_linear_gated_packin";
  convrot_status st = check_act(fn);
  if (st != CONVROT_OK) return st;
  int lg = 0, lu = 0;
  st = check_packin(what, X, xdt, ldx, M, w_gate, b_gate, Y, ydt, ldy, true, false, &lg);
  if (st != CONVROT_OK) return st;
  st = check_packin(what, X, xdt, ldx, M, w_up, b_up, Y, ydt, ldy, true, false, &lu);
  if (st != CONVROT_OK) return st;
  if (w_gate->rows != w_up->rows || w_gate->K != w_up->K)
    return fail(CONVROT_ERR_MISMATCH, "%s: gate is [%lld, %lld] but up is [%lld, %lld]", what,
                static_cast<long long>(w_gate->rows), static_cast<long long>(w_gate->K),
                static_cast<long long>(w_up->rows), static_cast<long long>(w_up->K));
  if (w_gate->rot.group != w_up->rot.group || w_gate->rot.kind != w_up->rot.kind ||
      w_gate->rot.signs != w_up->rot.signs)
    return fail(CONVROT_ERR_MISMATCH, "%s: gate and up were packed with different rotations", what);
  if (w_gate->layout != w_up->layout)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: gate and up weights must have the same layout", what);
  if (M == 0 || w_gate->rows == 0) return ok();
  const hipError_t e = convrot::launch_gemv_i8_gated_packin(
      X, ldx, lg, static_cast<convrot::RotKind>(w_gate->rot.kind), w_gate->rot.signs, w_gate->q, w_gate->ld,
      w_gate->scale, b_gate, w_up->q, w_up->ld, w_up->scale, b_up, static_cast<convrot::Act>(fn), M, w_gate->rows,
      w_gate->K, Y, static_cast<convrot::Elt>(ydt), ldy, static_cast<hipStream_t>(stream),
      w_gate->layout == CONVROT_LAYOUT_TILE16);
  return from_hip(e, what);
}

convrot_status convrot_linear_bf16(const void* X, int64_t ldx, const void* W, int64_t ldw, const float* bias,
                                   int64_t M, int64_t N, int64_t K, void* Y, convrot_dtype ydt, int64_t ldy,
                                   void* workspace, int64_t workspace_bytes, void* stream) {
  convrot_status st = check_k(K, int64_t{1} << 30);
  if (st != CONVROT_OK) return st;
  if (N < 0 || N > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "bad N");
  st = check_matrix("X", X, M, K, ldx, 2);
  if (st != CONVROT_OK) return st;
  st = check_matrix("W", W, N, K, ldw, 2);
  if (st != CONVROT_OK) return st;
  if (ydt != CONVROT_F32 && ydt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "convrot_linear_bf16: output must be CONVROT_F32 or CONVROT_BF16");
  st = check_matrix("Y", Y, M, N, ldy, elt_size(ydt), false);
  if (st != CONVROT_OK) return st;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)
    return fail(CONVROT_ERR_ALIGN, "bias must be 4-byte aligned");
  if (2 * ldx > kMaxLdBytes || 2 * ldw > kMaxLdBytes)
    return fail(CONVROT_ERR_INVALID_ARG, "leading dimension of X or W exceeds %lld bytes",
                static_cast<long long>(kMaxLdBytes));
  if (M == 0 || N == 0) return ok();
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_BF16, M, N, K));
    if (st != CONVROT_OK) return st;
  }
  const auto out = static_cast<convrot::Elt>(ydt);
  const auto s = static_cast<hipStream_t>(stream);
  const hipError_t e = M <= convrot::kGemvMaxRows
                           ? convrot::launch_gemv_bf16(X, ldx, W, ldw, bias, M, N, K, Y, out, ldy, workspace, s)
                           : convrot::launch_gemm_bf16(X, ldx, W, ldw, bias, M, N, K, Y, out, ldy, s);
  return from_hip(e, "convrot_linear_bf16");
}

convrot_status convrot_rotate(const void* X, convrot_dtype xdt, int64_t M, int64_t K, int64_t ldx, convrot_rot rot,
                              float* Xrot, int64_t ldr, void* stream) {
  int log2G = 0;
  convrot_status st = check_k(K, kMaxPackK);
  if (st != CONVROT_OK) return st;
  st = check_rot(rot, K, &log2G);
  if (st != CONVROT_OK) return st;
  if (xdt != CONVROT_F32 && xdt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "convrot_rotate: input must be CONVROT_F32 or CONVROT_BF16");
  st = check_matrix("X", X, M, K, ldx, elt_size(xdt));
  if (st != CONVROT_OK) return st;
  st = check_matrix("Xrot", Xrot, M, K, ldr, 4);
  if (st != CONVROT_OK) return st;
  if (M == 0) return ok();
  const hipError_t e = convrot::launch_pack_rows(X, static_cast<convrot::Elt>(xdt), M, K, ldx, log2G,
                                                 static_cast<convrot::RotKind>(rot.kind), rot.signs, nullptr, 0,
                                                 nullptr, Xrot, ldr, static_cast<hipStream_t>(stream));
  return from_hip(e, "convrot_rotate");
}

convrot_status convrot_pack_weight_w4(const void* W, convrot_dtype wdt, int64_t ldw, const convrot_packed_w4* out,
                                      void* stream) {
  const char* what = "convrot_pack_weight_w4";
  int log2G = 0;
  if (out == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: output descriptor is NULL", what);
  convrot_status st = check_k(out->K, kMaxPackK);
  if (st != CONVROT_OK) return st;
  st = check_packed_w4("packed output", out, &log2G);
  if (st != CONVROT_OK) return st;
  st = check_rows_layout("packed output", out->layout);
  if (st != CONVROT_OK) return st;
  if (wdt != CONVROT_F32 && wdt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "%s: input must be CONVROT_F32 or CONVROT_BF16", what);
  st = check_matrix("input", W, out->rows, out->K, ldw, elt_size(wdt));
  if (st != CONVROT_OK) return st;
  if (out->rows == 0) return ok();
  const hipError_t e = convrot::launch_pack_rows_w4(W, static_cast<convrot::Elt>(wdt), out->rows, out->K, ldw, log2G,
                                                    static_cast<convrot::RotKind>(out->rot.kind), out->rot.signs,
                                                    out->q, out->ld, out->scale, static_cast<hipStream_t>(stream));
  return from_hip(e, what);
}

convrot_status convrot_linear_w4(const convrot_packed* act, const convrot_packed_w4* w, const float* bias,
                                 convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  const char* what = "convrot_linear_w4";
  if (fn != CONVROT_ACT_NONE) {
    convrot_status st = check_act(fn);
    if (st != CONVROT_OK) return st;
  }
  int lg = 0;
  convrot_status st = check_packed_w4("weight", w, &lg);
  if (st != CONVROT_OK) return st;
  const convrot_packed wv = as_int8_view(*w);
  st = check_linear(what, act, &wv, bias, Y, ydt, ldy, fn == CONVROT_ACT_NONE);
  if (st == CONVROT_OK) st = check_rows_layout("activation", act->layout);
  if (st != CONVROT_OK) return st;
  const int64_t M = act->rows, N = w->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  const auto out = static_cast<convrot::Elt>(ydt);
  const auto a = static_cast<convrot::Act>(fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_W4, M, N, K));
    if (st != CONVROT_OK) return st;
    return from_hip(convrot::launch_gemv_w4(act->q, act->ld, w->q, w->ld, act->scale, w->scale, bias, a, M, N, K, Y,
                                            out, ldy, workspace, s, w->layout == CONVROT_LAYOUT_TILE16),
                    what);
  }
  st = check_workspace(workspace, workspace_bytes, N * K);
  if (st != CONVROT_OK) return st;
  int8_t* w8 = static_cast<int8_t*>(workspace);
  hipError_t e = convrot::launch_unpack_w4(w->q, w->ld, N, K, w8, K, s);
  if (e == hipSuccess) {
    e = fn == CONVROT_ACT_NONE
            ? convrot::launch_gemm_i8(act->q, act->ld, w8, K, act->scale, w->scale, bias, M, N, K, Y, out, ldy, s)
            : convrot::launch_gemm_i8_act(act->q, act->ld, w8, K, act->scale, w->scale, bias, a, M, N, K, Y, out,
                                          ldy, s);
  }
  return from_hip(e, what);
}

convrot_status convrot_linear_w4_gated(const convrot_packed* act, const convrot_packed_w4* w_gate,
                                       const float* b_gate, const convrot_packed_w4* w_up, const float* b_up,
                                       convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                       int64_t workspace_bytes, void* stream) {
  const char* what = "convrot_linear_w4_gated";
  convrot_status st = check_act(fn);
  if (st != CONVROT_OK) return st;
  int lg = 0;
  st = check_packed_w4("gate weight", w_gate, &lg);
  if (st != CONVROT_OK) return st;
  st = check_packed_w4("up weight", w_up, &lg);
  if (st != CONVROT_OK) return st;
  const convrot_packed gv = as_int8_view(*w_gate), uv = as_int8_view(*w_up);
  st = check_linear(what, act, &gv, b_gate, Y, ydt, ldy, false);
  if (st == CONVROT_OK) st = check_rows_layout("activation", act->layout);
  if (st != CONVROT_OK) return st;
  st = check_linear(what, act, &uv, b_up, Y, ydt, ldy, false);
  if (st != CONVROT_OK) return st;
  if (w_gate->rows != w_up->rows)
    return fail(CONVROT_ERR_MISMATCH, "gate has %lld output rows but up has %lld",
                static_cast<long long>(w_gate->rows), static_cast<long long>(w_up->rows));
  if (w_gate->layout != w_up->layout)
    return fail(CONVROT_ERR_INVALID_ARG, "convrot_linear_w4_gated: gate and up weights must have the same layout");
  const int64_t M = act->rows, N = w_gate->rows, K = act->K;
  if (M == 0 || N == 0) return ok();
  const auto out = static_cast<convrot::Elt>(ydt);
  const auto a = static_cast<convrot::Act>(fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= convrot::kGemvMaxRows) {
    st = check_split_workspace(workspace, workspace_bytes, small_m_workspace(CONVROT_LINEAR_W4_GATED, M, N, K));
    if (st != CONVROT_OK) return st;
    return from_hip(convrot::launch_gemv_w4_gated(act->q, act->ld, w_gate->q, w_gate->ld, w_gate->scale, b_gate,
                                                  w_up->q, w_up->ld, w_up->scale, b_up, act->scale, a, M, N, K, Y,
                                                  out, ldy, workspace, s, w_gate->layout == CONVROT_LAYOUT_TILE16),
                    what);
  }
  st = check_workspace(workspace, workspace_bytes, 2 * N * K);
  if (st != CONVROT_OK) return st;
  int8_t* g8 = static_cast<int8_t*>(workspace);
  int8_t* u8 = g8 + N * K;
  hipError_t e = convrot::launch_unpack_w4(w_gate->q, w_gate->ld, N, K, g8, K, s);
  if (e == hipSuccess) e = convrot::launch_unpack_w4(w_up->q, w_up->ld, N, K, u8, K, s);
  if (e == hipSuccess)
    e = convrot::launch_gemm_i8_gated(act->q, act->ld, g8, K, w_gate->scale, b_gate, u8, K, w_up->scale, b_up,
                                      act->scale, a, M, N, K, Y, out, ldy, s);
  return from_hip(e, what);
}

convrot_status convrot_unpack_w4(const convrot_packed_w4* w, int8_t* dst, int64_t ldd, void* stream) {
  int lg = 0;
  convrot_status st = check_packed_w4("weight", w, &lg);
  if (st != CONVROT_OK) return st;
  st = check_rows_layout("weight", w->layout);
  if (st != CONVROT_OK) return st;
  st = check_matrix("dst", dst, w->rows, w->K, ldd, 1);
  if (st != CONVROT_OK) return st;
  if (w->rows == 0) return ok();
  return from_hip(convrot::launch_unpack_w4(w->q, w->ld, w->rows, w->K, dst, ldd, static_cast<hipStream_t>(stream)),
                  "convrot_unpack_w4");
}

convrot_status convrot_tile_weight(const convrot_packed* in, const convrot_packed* out, void* stream) {
  if (in == nullptr || out == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "convrot_tile_weight: NULL descriptor");
  return tile_impl<convrot_packed>("convrot_tile_weight", in, out, in->K, stream, check_packed);
}

convrot_status convrot_tile_weight_w4(const convrot_packed_w4* in, const convrot_packed_w4* out, void* stream) {
  if (in == nullptr || out == nullptr)
    return fail(CONVROT_ERR_INVALID_ARG, "convrot_tile_weight_w4: NULL descriptor");
  return tile_impl<convrot_packed_w4>("convrot_tile_weight_w4", in, out, in->K / 2, stream, check_packed_w4);
}

convrot_status convrot_smooth_ffn(const void* W_up, convrot_dtype up_dt, int64_t ldu, const void* W_down,
                                  convrot_dtype down_dt, int64_t ldd, int64_t F, int64_t K, int64_t K_out,
                                  convrot_smooth_norm norm, float* s, float* W_up_out, int64_t ldu_out,
                                  float* W_down_out, int64_t ldd_out, void* stream) {
  const char* what = "convrot_smooth_ffn";
  if (F < 0 || K < 0 || K_out < 0 || F > kMaxRows || K_out > kMaxRows)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: bad sizes", what);
  if ((up_dt != CONVROT_F32 && up_dt != CONVROT_BF16) || (down_dt != CONVROT_F32 && down_dt != CONVROT_BF16))
    return fail(CONVROT_ERR_DTYPE, "%s: weights must be CONVROT_F32 or CONVROT_BF16", what);
  if (norm != CONVROT_SMOOTH_L2 && norm != CONVROT_SMOOTH_MAX)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: unknown norm %d", what, static_cast<int>(norm));
  if (F == 0) return ok();
  if (s == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "%s: s is NULL", what);
  if ((reinterpret_cast<uintptr_t>(s) & 3u) != 0) return fail(CONVROT_ERR_ALIGN, "s must be 4-byte aligned");
  convrot_status st = check_matrix("W_up", W_up, F, K, ldu, elt_size(up_dt), false);
  if (st != CONVROT_OK) return st;
  st = check_matrix("W_down", W_down, K_out, F, ldd, elt_size(down_dt), false);
  if (st != CONVROT_OK) return st;
  if (W_up_out != nullptr) {
    st = check_matrix("W_up_out", W_up_out, F, K, ldu_out, 4, false);
    if (st != CONVROT_OK) return st;
  }
  if (W_down_out != nullptr) {
    st = check_matrix("W_down_out", W_down_out, K_out, F, ldd_out, 4, false);
    if (st != CONVROT_OK) return st;
  }
  const hipError_t e = convrot::launch_smooth_ffn(
      W_up, static_cast<convrot::Elt>(up_dt), ldu, W_down, static_cast<convrot::Elt>(down_dt), ldd, F, K, K_out,
      norm == CONVROT_SMOOTH_MAX, s, W_up_out, ldu_out, W_down_out, ldd_out, static_cast<hipStream_t>(stream));
  return from_hip(e, what);
}

namespace {
// Workspace of the LoRA correction: bf16 T [M, r] first, then (when the down
// product splits K) the fp32 partials from the next 256-byte boundary.
int64_t lora_t_bytes(int64_t M, int64_t r) { return (2 * M * r + 255) / 256 * 256; }
int64_t lora_ws_bytes(int64_t M, int64_t K, int64_t r) {
  const int nb = convrot::lora_down_blocks(M, K, r);
  return lora_t_bytes(M, r) + (nb > 1 ? 4 * static_cast<int64_t>(nb) * M * r : 0);
}
convrot_status check_lora_shape(const char* what, int64_t M, int64_t K, int64_t r) {
  convrot_status st = check_k(K, int64_t{1} << 30);
  if (st != CONVROT_OK) return st;
  if (r <= 0 || r % 16 != 0 || r > 256)
    return fail(CONVROT_ERR_INVALID_ARG, "%s: rank r = %lld must be a positive multiple of 16, at most 256", what,
                static_cast<long long>(r));
  if (M < 0 || M > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "%s: bad M", what);
  return CONVROT_OK;
}
}  // namespace

convrot_status convrot_lora_workspace_bytes(int64_t M, int64_t K, int64_t r, int64_t* bytes) {
  if (bytes == nullptr) return fail(CONVROT_ERR_INVALID_ARG, "convrot_lora_workspace_bytes: bytes is NULL");
  const convrot_status st = check_lora_shape("convrot_lora_workspace_bytes", M, K, r);
  if (st != CONVROT_OK) return st;
  *bytes = M == 0 ? 0 : lora_ws_bytes(M, K, r);
  return ok();
}

convrot_status convrot_lora_add(const void* X, int64_t ldx, int64_t M, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, int64_t N, int64_t r, float scale, void* Y,
                                convrot_dtype ydt, int64_t ldy, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  const char* what = "convrot_lora_add";
  convrot_status st = check_lora_shape(what, M, K, r);
  if (st != CONVROT_OK) return st;
  if (N < 0 || N > kMaxRows) return fail(CONVROT_ERR_INVALID_ARG, "%s: bad N", what);
  if (ydt != CONVROT_F32 && ydt != CONVROT_BF16)
    return fail(CONVROT_ERR_DTYPE, "%s: Y must be CONVROT_F32 or CONVROT_BF16", what);
  st = check_matrix("X", X, M, K, ldx, 2);
  if (st != CONVROT_OK) return st;
  st = check_matrix("A", A, r, K, lda, 2);
  if (st != CONVROT_OK) return st;
  st = check_matrix("B", B, N, r, ldb, 2);
  if (st != CONVROT_OK) return st;
  st = check_matrix("Y", Y, M, N, ldy, elt_size(ydt), false);
  if (st != CONVROT_OK) return st;
  if (2 * ldx > kMaxLdBytes || 2 * lda > kMaxLdBytes)
    return fail(CONVROT_ERR_INVALID_ARG, "leading dimension of X or A exceeds %lld bytes",
                static_cast<long long>(kMaxLdBytes));
  if (M == 0 || N == 0) return ok();
  st = check_workspace(workspace, workspace_bytes, lora_ws_bytes(M, K, r));
  if (st != CONVROT_OK) return st;
  const auto s = static_cast<hipStream_t>(stream);
  auto* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + lora_t_bytes(M, r));
  hipError_t e = convrot::launch_lora_down(X, ldx, A, lda, M, K, r, workspace, r, partials, s);
  if (e == hipSuccess)
    e = convrot::launch_lora_up(workspace, r, B, ldb, M, N, r, scale, Y, static_cast<convrot::Elt>(ydt), ldy, s);
  return from_hip(e, what);
}

const char* convrot_status_string(convrot_status status) {
  switch (status) {
    case CONVROT_OK: return "CONVROT_OK";
    case CONVROT_ERR_INVALID_ARG: return "CONVROT_ERR_INVALID_ARG";
    case CONVROT_ERR_GROUP: return "CONVROT_ERR_GROUP";
    case CONVROT_ERR_DTYPE: return "CONVROT_ERR_DTYPE";
    case CONVROT_ERR_ALIGN: return "CONVROT_ERR_ALIGN";
    case CONVROT_ERR_MISMATCH: return "CONVROT_ERR_MISMATCH";
    case CONVROT_ERR_HIP: return "CONVROT_ERR_HIP";
  }
  return "unknown convrot_status";
}

const char* convrot_last_error(void) { return g_last_error; }

int convrot_abi_version(void) { return CONVROT_ABI_VERSION; }

}  // extern "C"
