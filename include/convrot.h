/*
 * convrot.h -- C ABI of the MI355X (gfx950) INT8 ConvRot W8A8 linear layer.
 *
 * The method (stable-diffusion.cpp documentation page "INT8 Convrot
 * Safetensors", sections "How INT8 convrot works", "Weight quantization" and
 * "Runtime activation quantization"):
 *
 *   R        block-diagonal rotation; every contiguous group of G input
 *            features is multiplied by the normalised Kronecker power of the
 *            4x4 regular Hadamard matrix H4 (G = 4^n).  R is orthogonal and
 *            symmetric.
 *   W_rot  = W R          (offline)      X_rot = X R          (run time)
 *   s[r]   = max_i |rot[r, i]| / 127     one scale per row (weights: per
 *                                        output row; activations: per row,
 *                                        computed at run time)
 *   Q[r,i] = clamp(round(rot[r, i] / s[r]), -127, 127)
 *   A[r,o] = sum_i Qx[r, i] * Qw[o, i]   exact signed 32-bit accumulation
 *   Y[r,o] = A[r, o] * s_x[r] * s_w[o] + b[o]
 *
 * One packed activation (Qx, s_x) serves every linear layer that shares the
 * same input and the same rotation (same page, "Runtime activation
 * quantization", last paragraph).
 *
 * A second rotation kind follows the gemma.cpp issue "Add experimental W8A8
 * MatMul with optional QuaRot-style rotation", section "Rotation method":
 * each block of G features is multiplied elementwise by fixed +-1 signs,
 * then by the natural-order (Sylvester) Walsh-Hadamard matrix, then by
 * 1/sqrt(G); the same transform is applied to activation rows and to weight
 * rows.
 *
 * Layers whose input width K is not a multiple of G stay unquantised (sglang
 * PR 34581 summary page, implementation section on kitchen_int8 routing);
 * convrot_linear_bf16 is that path.  The library never falls back silently:
 * routing is the caller's decision.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device,
 *   row-major, with explicit leading dimensions counted in ELEMENTS of the
 *   tensor's own type.  Every input matrix (X, W, packed codes) and every
 *   output of the pack and rotate entry points must have a 16-byte aligned
 *   base and a leading dimension whose size in bytes is a multiple of 16.
 *   The Y output of the linear entry points only needs element alignment.
 * - The caller owns every buffer, inputs, outputs and workspaces alike.
 *   The library allocates no device memory.  Its only state is a
 *   thread-local error string and, per device, the CU count and the kernel
 *   attributes it has set (written once, never reset).
 * - Workspaces.  The linear entry points take `workspace` (a device pointer,
 *   16-byte aligned, or NULL) and `workspace_bytes`.  With M <= 16 a
 *   workspace of convrot_linear_workspace_bytes(...) bytes lets the
 *   weight-streaming kernel split K across workgroups when the output has
 *   fewer 16-feature tiles than the GPU has CUs: the partial sums go there
 *   and a second launch adds them in K order.  NULL selects the unsplit
 *   kernel.  int8 results are the same bits either way; bf16 results of
 *   convrot_linear_bf16 may differ in the last place (fp32 summation
 *   order).  A non-NULL workspace smaller than the query's size is
 *   CONVROT_ERR_INVALID_ARG.  The int4 entry points with M > 16 need one
 *   (the expanded weight).  A call fully rewrites what it uses, so a
 *   workspace needs no clearing and captured graphs may replay such calls.
 *   Calls that may run at the same time (different streams) need separate
 *   workspaces.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL selects the
 *   default stream).  Inputs must stay alive, and outputs untouched, until
 *   the stream has passed the call.  Outputs must not alias inputs.
 * - Validation happens on the host before anything is enqueued.  On any
 *   error the call enqueues nothing, leaves outputs untouched and returns a
 *   non-zero status; convrot_last_error() then describes it.  A launch that
 *   the HIP runtime rejects returns CONVROT_ERR_HIP.
 * - Empty problems (M == 0 or N == 0) return CONVROT_OK and launch nothing.
 * - K must be a positive multiple of 16 (the kernels move 16-byte chunks).
 * - Non-finite inputs are outside the method's domain; results are then
 *   unspecified (no fault, no error).
 * - No exception crosses this boundary.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_ABI_VERSION 10

typedef enum {
  CONVROT_OK = 0,
  CONVROT_ERR_INVALID_ARG = 1, /* null pointer, negative size, K % 16 != 0, bad leading dimension */
  CONVROT_ERR_GROUP = 2,       /* G not allowed for the rotation kind, or K % G != 0 */
  CONVROT_ERR_DTYPE = 3,       /* element type not accepted by this entry point */
  CONVROT_ERR_ALIGN = 4,       /* base pointer not 16-byte aligned, or ld * elt % 16 != 0 */
  CONVROT_ERR_MISMATCH = 5,    /* activation and weight packed with different K or rotation */
  CONVROT_ERR_HIP = 6          /* the HIP runtime rejected a launch */
} convrot_status;

typedef enum {
  CONVROT_F32 = 0,
  CONVROT_BF16 = 1,
  CONVROT_I32 = 2 /* raw accumulator A (convrot_linear output only; for checking) */
} convrot_dtype;

typedef enum {
  /* "INT8 Convrot Safetensors": R_G = normalised H4^{(x)n}, G = 4^n in {4, 16, 64, 256, 1024}. */
  CONVROT_ROT_REGULAR = 0,
  /* gemma.cpp issue, "Rotation method": (1/sqrt G) H_sylvester D, G = 2^m in {16, 32, ..., 1024}. */
  CONVROT_ROT_RANDOMIZED = 1
} convrot_rot_kind;

/* Activation applied by a fused epilogue (convrot_linear_act,
 * convrot_linear_gated):
 *   GELU_ERF   gelu(y) = y Phi(y) = y/2 (1 + erf(y / sqrt 2)), with the
 *              normal tail 1 - Phi(|y|) from the five-term erfc
 *              approximation of Abramowitz & Stegun, formula 7.1.26
 *              (absolute error <= 1.5e-7 on erfc, so |gelu error| <=
 *              7.5e-8 |y| before fp32 rounding), evaluated with the
 *              hardware reciprocal and exp2
 *   GELU_TANH  gelu(y) = y/2 (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3),
 *              evaluated as y / (1 + exp(-2u)) with the hardware exp2 and
 *              reciprocal (a few fp32 ulp of y)  */
typedef enum {
  CONVROT_ACT_NONE = 0, /* not accepted by the fused entry points (use convrot_linear) */
  CONVROT_ACT_GELU_ERF = 1,
  CONVROT_ACT_GELU_TANH = 2
} convrot_act;

/* Which linear entry point a workspace query is for
 * (convrot_linear_workspace_bytes). */
typedef enum {
  CONVROT_LINEAR_PLAIN = 0,    /* convrot_linear, convrot_linear_act */
  CONVROT_LINEAR_GATED = 1,    /* convrot_linear_gated */
  CONVROT_LINEAR_BF16 = 2,     /* convrot_linear_bf16 */
  CONVROT_LINEAR_W4 = 3,       /* convrot_linear_w4 */
  CONVROT_LINEAR_W4_GATED = 4  /* convrot_linear_w4_gated */
} convrot_linear_kind;

/* Norm of the data-free smoothing scales (convrot_smooth_ffn). */
typedef enum {
  CONVROT_SMOOTH_L2 = 0, /* s_j = sqrt(||W_up[j, :]||_2 / ||W_down[:, j]||_2) */
  CONVROT_SMOOTH_MAX = 1 /* the same with the largest magnitudes */
} convrot_smooth_norm;

/* Rotation descriptor.  `signs` is a device vector of K int8 values, each +1
 * or -1 (one sign per input feature, block b using signs[b*G .. b*G+G-1]);
 * it is required for CONVROT_ROT_RANDOMIZED and must be NULL otherwise. */
typedef struct {
  int32_t group;        /* G */
  int32_t kind;         /* convrot_rot_kind */
  const int8_t* signs;  /* [K] +-1, randomized kind only */
} convrot_rot;

/* Where a packed operand's codes lie in memory (the `layout` field of
 * convrot_packed and convrot_packed_w4).
 *   ROWS    row-major [rows, ld], as described with each struct (the
 *           checkpoint layout; every entry point reads it).
 *   TILE16  rows grouped in tiles of 16 consecutive rows and, within a
 *           tile, K cut into units of 64 bytes (64 int8 codes or 128 int4
 *           codes); with ld equal to the bytes of one row (K, or K / 2 for
 *           int4), byte b of row r is at
 *             q + (r / 16) * 16 * ld + (b / 64) * 1024 + (r % 16) * 64 + b % 64
 *           so the 16 rows' bytes of one unit are 1 KiB of consecutive
 *           memory, which the weight-streaming kernel (M <= 16) reads
 *           faster than 16 row pieces 1 row apart.  Only that path reads
 *           it: a linear call with a TILE16 weight and M > 16 is
 *           CONVROT_ERR_INVALID_ARG.  It needs rows % 16 == 0, ld == the row
 *           bytes, and K % 64 == 0 (int4: K % 128 == 0).
 *           convrot_tile_weight and convrot_tile_weight_w4 convert a ROWS
 *           weight.
 *           A packed activation may take it as well (the same formula;
 *           ld == K, K % 64 == 0, any row count, the buffer holding whole
 *           tiles of 16 rows, i.e. 16 K bytes for M <= 16): the
 *           activation fragments of the weight-streaming kernel are then
 *           1 KiB of consecutive memory per unit instead of 16 row pieces
 *           (measured: decode step 3.5-5% faster at M = 4-16, level at M = 1).  convrot_pack_act
 *           writes it when its output descriptor asks for it; convrot_linear,
 *           _act, _gated and _noalloc read it for M <= 16 with int8 weights
 *           of either layout; every other entry point takes ROWS
 *           activations (CONVROT_ERR_INVALID_ARG otherwise). */
typedef enum {
  CONVROT_LAYOUT_ROWS = 0,
  CONVROT_LAYOUT_TILE16 = 1
} convrot_layout;

/* A packed operand: int8 rows and one fp32 scale per row, both caller-owned
 * device buffers, plus the rotation that produced them.
 *   q      [rows, ld] int8, row-major, ld >= K, ld % 16 == 0 (or the TILE16
 *          layout above)
 *   scale  [rows] fp32
 *   layout convrot_layout
 * The same struct describes a packed activation (rows = M) and a packed
 * weight (rows = N; the canonical checkpoint layout, one int8 row per output
 * feature, "INT8 Convrot Safetensors", "Checkpoint format"). */
typedef struct {
  int8_t* q;
  float* scale;
  int64_t rows;
  int64_t K;
  int64_t ld;
  convrot_rot rot;
  int32_t layout;
} convrot_packed;

/* A packed int4 weight (W4A8; stable-diffusion.cpp PR "load ConvRot int4 and
 * per-channel int8 safetensors", sections "Solution" and "The rotation"):
 * the rotated weight W R quantised to codes in [-7, 7] with one fp32 scale
 * per output row (row max / 7), two codes per byte.
 *   q      [rows, ld] bytes, row-major; byte j of a row holds element 2j in
 *          its low nibble and element 2j + 1 in its high nibble, each as
 *          4-bit two's complement; ld >= K / 2 and ld % 8 == 0 (bytes; the rows
 *          are read in 8-byte units), q 16-byte aligned
 *   scale  [rows] fp32
 * Both buffers are caller-owned device memory. */
typedef struct {
  uint8_t* q;
  float* scale;
  int64_t rows;
  int64_t K;
  int64_t ld;
  convrot_rot rot;
  int32_t layout;  /* convrot_layout */
} convrot_packed_w4;

/* Rotate and quantise activation rows ("Runtime activation quantization").
 *   X     [out->rows, ldx] of `xdt` (CONVROT_F32 or CONVROT_BF16), K = out->K
 *   out   descriptor of the caller-owned destination; out->q and out->scale
 *         are written, the struct itself is not modified.
 * One fused kernel: group-wise Hadamard rotation, whole-row absmax, rounding
 * to nearest even and clamping to [-127, 127].  An all-zero row gets scale 0
 * and zero codes.  Deterministic: the same input gives the same bits. */
convrot_status convrot_pack_act(const void* X, convrot_dtype xdt, int64_t ldx,
                                const convrot_packed* out, void* stream);

/* Rotate and quantise weight rows ("Weight quantization"): the same
 * transform and rule as convrot_pack_act, one scale per output row.  Runs
 * once, offline, on W [out->rows = N, K]. */
convrot_status convrot_pack_weight(const void* W, convrot_dtype wdt, int64_t ldw,
                                   const convrot_packed* out, void* stream);

/* The quantised linear ("Runtime activation quantization"):
 *   Y[r, o] = A[r, o] * act->scale[r] * w->scale[o] + bias[o]
 * with A the exact int32 product of act->q and w->q^T.
 *   act   packed activation [M = act->rows, K]
 *   w     packed weight [N = w->rows, K]; act->K == w->K and the two
 *         rotation descriptors must be equal (same G, kind and signs
 *         pointer), otherwise CONVROT_ERR_MISMATCH; ROWS layout, or TILE16
 *         when M <= 16 (CONVROT_ERR_INVALID_ARG otherwise)
 *   bias  [N] fp32 or NULL
 *   Y     [M, ldy] of `ydt`: CONVROT_F32, CONVROT_BF16 (round to nearest
 *         even) or CONVROT_I32 (the raw accumulator A; scales and bias are
 *         then not applied)
 *   workspace, workspace_bytes
 *         NULL / 0, or caller-owned device memory of at least
 *         convrot_linear_workspace_bytes(CONVROT_LINEAR_PLAIN, M, N, K)
 *         bytes (see "Workspaces" above)
 * Small M (<= 16) uses a weight-streaming kernel, larger M a tiled
 * matrix-core kernel; both produce bit-identical A (the small-M kernel's
 * split over K adds exact int32 partial sums). */
convrot_status convrot_linear(const convrot_packed* act, const convrot_packed* w,
                              const float* bias, void* Y, convrot_dtype ydt, int64_t ldy,
                              void* workspace, int64_t workspace_bytes, void* stream);

/* Size of the static scratch of convrot_linear_noalloc (bytes). */
#define CONVROT_NOALLOC_SCRATCH_BYTES (1 << 20)

/* convrot_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks, kernels and result bits as
 * convrot_linear with a workspace, but the small-M split's partial sums go
 * to a static device array of CONVROT_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends.  Nothing is
 * allocated, by the library or on its behalf.
 *   - A shape whose split needs more than that scratch is rejected with
 *     CONVROT_ERR_INVALID_ARG before anything is enqueued (on a 256-CU GPU
 *     the largest split of this entry point needs 0.75 MiB, so every shape
 *     fits there).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's partial sums; each call fully rewrites what it reads, so
 *     nothing needs clearing.  Calls that overlap in time on one GPU
 *     (different streams, or graphs replayed concurrently) race on it and
 *     give wrong results; calls ordered on one stream or by events do not.
 *   - The scratch's device address is resolved on the first call on each
 *     device (hipGetSymbolAddress); a failure there is CONVROT_ERR_HIP. */
convrot_status convrot_linear_noalloc(const convrot_packed* act, const convrot_packed* w, const float* bias, void* Y,
                                      convrot_dtype ydt, int64_t ldy, void* stream);

/* Bytes of workspace a linear call of `kind` uses for X [M, K] and N
 * outputs on the current device:
 *   M <= 16  the split-K partial sums (0 when the shape does not split K;
 *            always 0 for the int4 kinds, whose split measured slower, and
 *            for plain int8 calls with M <= 12, which run one wide
 *            workgroup per tile instead; with a TILE16 activation plain
 *            int8 calls up to M = 16 take the wide workgroups too and leave
 *            the workspace unused); optional, NULL selects the unsplit
 *            kernel
 *   M > 16   0, except CONVROT_LINEAR_W4 (N * K, required) and
 *            CONVROT_LINEAR_W4_GATED (2 * N * K, required)
 * The size depends on the device's CU count.  M, N >= 0 and K a positive
 * multiple of 16, else CONVROT_ERR_INVALID_ARG. */
convrot_status convrot_linear_workspace_bytes(convrot_linear_kind kind, int64_t M, int64_t N, int64_t K,
                                              int64_t* bytes);

/* The quantised linear with an activation fused into its epilogue (the
 * output of the linear is never written unactivated):
 *   Y[r, o] = fn(A[r, o] * act->scale[r] * w->scale[o] + bias[o])
 * Arguments, checks and errors as convrot_linear, plus:
 *   fn    CONVROT_ACT_GELU_ERF or CONVROT_ACT_GELU_TANH, else
 *         CONVROT_ERR_INVALID_ARG
 *   ydt   CONVROT_F32 or CONVROT_BF16 (CONVROT_I32 is rejected with
 *         CONVROT_ERR_DTYPE).
 *   workspace, workspace_bytes  as convrot_linear (kind CONVROT_LINEAR_PLAIN)
 * A packed activation feeds the next layer's linear; this entry point is
 * for a layer followed by an activation, such as the first linear of an
 * MLP. */
convrot_status convrot_linear_act(const convrot_packed* act, const convrot_packed* w, const float* bias,
                                  convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/* Producer fusion of the next layer's pack.  The activation side of the
 * method is a rotation, a whole-row maximum and a quantisation ("INT8
 * Convrot Safetensors", "Backend support" and "Runtime activation
 * quantization": the row's scale is its largest rotated magnitude over 127).
 * This is convrot_linear_act that, in the same launch, also computes the
 * row maximum's parts for the layer that reads Y: for every row r of Y and
 * every contiguous group j of group_next output features,
 *   rowmax[r, j] = max over the group of |(Y[r, group j] R)_i|
 * with R the regular rotation of size group_next, applied to Y as stored
 * (a bf16 Y is rounded first).  convrot_pack_act_rowmax then packs Y with
 * these maxima and skips its own row reduction; the codes and scales are
 * those of convrot_pack_act on Y, bit for bit (both evaluate the rotation
 * with the same operations in the same order).
 *   group_next  4, 16, 64 or 256, else CONVROT_ERR_GROUP
 *   rowmax      [M, ldm] fp32, caller-owned, 4-byte aligned,
 *               ldm >= N / group_next
 * Needs M > 16 (the tiled kernel), N % 256 == 0, K % 128 == 0 and Y rows
 * aligned for 4-element stores (Y aligned to 4 elements, ldy % 4 == 0);
 * otherwise CONVROT_ERR_INVALID_ARG.  Other arguments, checks and errors as
 * convrot_linear_act. */
convrot_status convrot_linear_act_rowmax(const convrot_packed* act, const convrot_packed* w, const float* bias,
                                         convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, int32_t group_next,
                                         float* rowmax, int64_t ldm, void* stream);

/* The pack of activation rows whose rotated group maxima are given (as
 * convrot_linear_act_rowmax writes them): the codes and scales of
 * convrot_pack_act, with the row maximum taken from `rowmax` instead of a
 * reduction over the row.
 *   X       [out->rows, ldx] of `xdt` (CONVROT_F32 or CONVROT_BF16)
 *   rowmax  [out->rows, ldm] fp32, ldm >= K / G, the maxima for
 *           G = out->rot.group
 *   out     as convrot_pack_act; the rotation must be the regular kind with
 *           G in {4, 16, 64, 256} (else CONVROT_ERR_GROUP)
 * Maxima that do not belong to X give a wrong scale; nothing checks them. */
convrot_status convrot_pack_act_rowmax(const void* X, convrot_dtype xdt, int64_t ldx, const float* rowmax,
                                       int64_t ldm, const convrot_packed* out, void* stream);

/* A gated pair: two quantised linears that share one packed activation,
 * combined in the epilogue of a single launch,
 *   G[r, o] = A_gate[r, o] * act->scale[r] * w_gate->scale[o] + b_gate[o]
 *   U[r, o] = A_up[r, o]   * act->scale[r] * w_up->scale[o]   + b_up[o]
 *   Y[r, o] = fn(G[r, o]) * U[r, o]
 * (the gated feed-forward layer; "INT8 Convrot Safetensors", "Runtime
 * activation quantization", last paragraph: one packed activation for
 * every linear that shares the input).
 *   w_gate, w_up  packed weights [N, K], each checked against `act` as in
 *                 convrot_linear; they must have the same N
 *                 (CONVROT_ERR_MISMATCH otherwise) and the same layout
 *                 (CONVROT_ERR_INVALID_ARG otherwise)
 *   b_gate, b_up  [N] fp32 or NULL
 *   fn, ydt       as convrot_linear_act
 *   Y             [M, ldy]
 *   workspace, workspace_bytes  as convrot_linear (kind
 *                 CONVROT_LINEAR_GATED). */
convrot_status convrot_linear_gated(const convrot_packed* act, const convrot_packed* w_gate, const float* b_gate,
                                    const convrot_packed* w_up, const float* b_up, convrot_act fn, void* Y,
                                    convrot_dtype ydt, int64_t ldy, void* workspace, int64_t workspace_bytes,
                                    void* stream);

/* Few-row linears that pack their own activation rows: the rotation, row
 * maximum and quantisation of convrot_pack_act ("INT8 Convrot Safetensors",
 * "Runtime activation quantization"; "Backend support" on fusing the three)
 * done inside the weight-streaming launch, every workgroup packing the rows
 * into on-chip memory with the pack kernel's operations, then the linear of
 * convrot_linear_act (plain) or convrot_linear_gated on those codes, all in
 * one launch.  The result bits equal packing with convrot_pack_act and then
 * calling convrot_linear / convrot_linear_act / convrot_linear_gated; the
 * packed rows are not written out.  For decoding, where the two launches'
 * fixed costs dominate.
 *   X       [M, ldx] bf16, rows 16-byte aligned (ldx * 2 a multiple of 16);
 *           other dtypes are CONVROT_ERR_DTYPE (pack them with
 *           convrot_pack_act)
 *   M       0 to 4 rows (more: CONVROT_ERR_INVALID_ARG)
 *   w       packed weight [N, K] (either layout); its rotation (G, kind,
 *           signs) is the one applied to X.  K at most 16384 for
 *           convrot_linear_packin and 4096 for convrot_linear_gated_packin
 *           (CONVROT_ERR_INVALID_ARG above)
 *   bias    [N] fp32 or NULL
 *   fn      CONVROT_ACT_NONE, _GELU_ERF or _GELU_TANH (plain); a GELU form
 *           (gated)
 *   Y       [M, ldy] of ydt: CONVROT_F32 or CONVROT_BF16, or CONVROT_I32
 *           (the raw accumulator) for the plain form without activation
 * The gated form takes w_gate and w_up as convrot_linear_gated does (same N,
 * K, rotation and layout: CONVROT_ERR_MISMATCH / CONVROT_ERR_INVALID_ARG).
 * Needs no workspace.  M = 0 or N = 0 launches nothing. */
convrot_status convrot_linear_packin(const void* X, convrot_dtype xdt, int64_t ldx, int64_t M, const convrot_packed* w,
                                     const float* bias, convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy,
                                     void* stream);
convrot_status convrot_linear_gated_packin(const void* X, convrot_dtype xdt, int64_t ldx, int64_t M,
                                           const convrot_packed* w_gate, const float* b_gate,
                                           const convrot_packed* w_up, const float* b_up, convrot_act fn, void* Y,
                                           convrot_dtype ydt, int64_t ldy, void* stream);

/* The unquantised path for layers the rotation cannot cover (K % G != 0):
 *   Y[r, o] = sum_i X[r, i] W[o, i] + bias[o]
 * bf16 operands, fp32 accumulation, output CONVROT_BF16 or CONVROT_F32.
 *   X [M, ldx] bf16, W [N, ldw] bf16, bias [N] fp32 or NULL, Y [M, ldy]
 *   workspace, workspace_bytes  as convrot_linear (kind CONVROT_LINEAR_BF16);
 *   with the split the fp32 partial sums are added in K order. */
convrot_status convrot_linear_bf16(const void* X, int64_t ldx, const void* W, int64_t ldw,
                                   const float* bias, int64_t M, int64_t N, int64_t K,
                                   void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/* The rotation alone, for checking: the same kernel as convrot_pack_act with
 * quantisation switched off, writing the fp32 rotated rows X R.
 *   X [M, ldx] of `xdt`, Xrot [M, ldr] fp32. */
convrot_status convrot_rotate(const void* X, convrot_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                              convrot_rot rot, float* Xrot, int64_t ldr, void* stream);

/* Rotate, quantise to int4 and pack weight rows offline: the transform of
 * convrot_pack_weight, then s = row max / 7 and codes rounded to nearest
 * even and clamped to [-7, 7], written as nibble pairs.  Arguments, checks
 * and errors as convrot_pack_weight, with `out` an int4 descriptor. */
convrot_status convrot_pack_weight_w4(const void* W, convrot_dtype wdt, int64_t ldw, const convrot_packed_w4* out,
                                      void* stream);

/* W4A8 linear: int8 activation codes against int4 weight codes,
 *   Y[r, o] = fn(A[r, o] * act->scale[r] * w->scale[o] + bias[o]),
 *   A = act->q (expanded w->q)^T, exact int32
 * (the same accumulation and epilogue as convrot_linear and
 * convrot_linear_act).
 *   act        packed activation [M, K]; act->K == w->K and equal rotation
 *              descriptors, else CONVROT_ERR_MISMATCH
 *   w          packed int4 weight [N, K]; ROWS layout, or TILE16 when
 *              M <= 16 (CONVROT_ERR_INVALID_ARG otherwise)
 *   fn         CONVROT_ACT_NONE (plain linear; ydt may then also be
 *              CONVROT_I32, the raw accumulator), CONVROT_ACT_GELU_ERF or
 *              CONVROT_ACT_GELU_TANH
 *   workspace  M <= 16: optional split-K partial sums as for
 *              convrot_linear (kind CONVROT_LINEAR_W4); the weight-streaming
 *              kernel reads the nibbles (half the bytes of an int8 weight)
 *              and expands them in registers.  M > 16: caller-owned device
 *              memory of at least workspace_bytes >= N * K bytes, 16-byte
 *              aligned, not shared with a concurrent call; the weight is
 *              expanded there to int8 codes and the tiled kernel runs.  Too
 *              small or NULL: CONVROT_ERR_INVALID_ARG. */
convrot_status convrot_linear_w4(const convrot_packed* act, const convrot_packed_w4* w, const float* bias,
                                 convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Gated pair with int4 weights, Y = fn(G) * U as in convrot_linear_gated;
 * fn must be CONVROT_ACT_GELU_ERF or CONVROT_ACT_GELU_TANH.  For M > 16 the
 * workspace holds both expanded weights: workspace_bytes >= 2 * N * K; for
 * M <= 16 it is optional, as for convrot_linear (kind
 * CONVROT_LINEAR_W4_GATED). */
convrot_status convrot_linear_w4_gated(const convrot_packed* act, const convrot_packed_w4* w_gate,
                                       const float* b_gate, const convrot_packed_w4* w_up, const float* b_up,
                                       convrot_act fn, void* Y, convrot_dtype ydt, int64_t ldy, void* workspace,
                                       int64_t workspace_bytes, void* stream);

/* Expand int4 codes to int8 codes (for checking, or to keep an int8 copy):
 *   w   ROWS layout
 *   dst [w->rows, ldd] int8, ldd >= w->K, ldd % 16 == 0, 16-byte aligned. */
convrot_status convrot_unpack_w4(const convrot_packed_w4* w, int8_t* dst, int64_t ldd, void* stream);

/* Copy a packed weight into the TILE16 layout (offline; see convrot_layout).
 *   in   packed weight in the ROWS layout (any valid ld)
 *   out  destination: layout CONVROT_LAYOUT_TILE16, the same rows, K and
 *        rotation as `in`, ld == K; out->q receives the rows * K code bytes
 *        in the tiled order and out->scale a copy of the scales.
 * Errors: CONVROT_ERR_INVALID_ARG for a wrong layout, rows % 16 != 0,
 * K % 64 != 0 or out->ld != K; CONVROT_ERR_MISMATCH when rows, K or the
 * rotation differ.  `in` and `out` must not overlap. */
convrot_status convrot_tile_weight(const convrot_packed* in, const convrot_packed* out, void* stream);

/* The same for int4 weights: out->ld == K / 2 and K % 128 == 0. */
convrot_status convrot_tile_weight_w4(const convrot_packed_w4* in, const convrot_packed_w4* out, void* stream);

/* Data-free smoothing of an FFN's intermediate channels, offline, before
 * the weights are packed (gemma.cpp issue "Add experimental W8A8 MatMul with
 * optional QuaRot-style rotation", the maintainer's review comment: scaling
 * without calibration data, by max norms or by the square root of the ratio
 * of the W_up to W_down L2 column norms, pulled into the per-row scales).
 * For channel j (row j of W_up, column j of W_down):
 *   s[j]           = sqrt(n_up[j] / n_down[j]), 1 where either norm is 0
 *   W_up_out[j, :] = W_up[j, :] / s[j],   W_down_out[:, j] = W_down[:, j] * s[j]
 * Norms accumulate in fp64; s is rounded once to fp32; each output weight is
 * the fp64 quotient or product with that s, rounded once to fp32.  Exact
 * for a gated FFN (h = act(gate) * up); the scaled weights are then packed
 * with convrot_pack_weight or convrot_pack_weight_w4.
 *   W_up      [F, ldu] of up_dt (CONVROT_F32 or CONVROT_BF16), K columns
 *   W_down    [K_out, ldd] of down_dt, F columns
 *   s         [F] fp32 (written)
 *   W_up_out  [F, ldu_out] fp32, or NULL to skip
 *   W_down_out [K_out, ldd_out] fp32, or NULL to skip
 * Only element alignment is required.  F == 0 is a no-op. */
convrot_status convrot_smooth_ffn(const void* W_up, convrot_dtype up_dt, int64_t ldu, const void* W_down,
                                  convrot_dtype down_dt, int64_t ldd, int64_t F, int64_t K, int64_t K_out,
                                  convrot_smooth_norm norm, float* s, float* W_up_out, int64_t ldu_out,
                                  float* W_down_out, int64_t ldd_out, void* stream);

/* Runtime LoRA correction added to a linear's output ("INT8 Convrot
 * Safetensors", LoRA paragraph: adapters are applied at run time without
 * touching the int8 weights; the correction is computed from the original,
 * unrotated activation and added to the base output):
 *   T = X A^T                 fp32 accumulation (in an unspecified order),
 *                             held in bf16
 *   Y[m, n] += scale * sum_j T[m, j] B[n, j]   (fp32 sum, one fused
 *                             multiply-add into Y; bf16 Y rounded to
 *                             nearest even)
 *   X   [M, ldx] bf16, the layer's unrotated input (K columns)
 *   A   [r, lda] bf16 (adapter down), B [N, ldb] bf16 (adapter up, r columns)
 *   r   rank, a positive multiple of 16, at most 256; K a positive multiple
 *       of 16
 *   Y   [M, ldy] of ydt (CONVROT_F32 or CONVROT_BF16), read and written
 *   workspace  caller-owned device memory, 16-byte aligned, of at least
 *       convrot_lora_workspace_bytes(M, K, r) bytes; not shared with a
 *       concurrent call.  T [M, r] bf16 is left at its start.
 * X, A, B: 16-byte aligned bases and rows.  Two or three launches on
 * `stream`: the down product into the workspace (split over K when the rows
 * alone give fewer workgroups than CUs, with a reduction of the fp32 block
 * partials in block order), then the up product with the add.  A smaller
 * workspace is CONVROT_ERR_INVALID_ARG.  A layer whose output goes through a
 * fused activation must run the plain linear, this call, and the activation
 * afterwards. */
/* Workspace bytes convrot_lora_add needs for X [M, K] and rank r on the
 * current device (0 when M == 0); the same argument checks as that call.
 * The size depends on the device's CU count through the K split. */
convrot_status convrot_lora_workspace_bytes(int64_t M, int64_t K, int64_t r, int64_t* bytes);

convrot_status convrot_lora_add(const void* X, int64_t ldx, int64_t M, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, int64_t N, int64_t r, float scale, void* Y,
                                convrot_dtype ydt, int64_t ldy, void* workspace, int64_t workspace_bytes,
                                void* stream);

/* Static description of a status code. */
const char* convrot_status_string(convrot_status status);

/* Description of the last error returned on the calling thread ("" if the
 * last call succeeded). */
const char* convrot_last_error(void);

/* CONVROT_ABI_VERSION of the built library. */
int convrot_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
