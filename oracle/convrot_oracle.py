"""CPU oracle for the INT8 ConvRot W8A8 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it.

It is a plain, slow, obviously correct numpy restatement of what the sources
define, written from the formulas:

* "INT8 Convrot Safetensors" (stable-diffusion.cpp docs), section
  "How INT8 convrot works": the normalised H4 matrix, its Kronecker power for
  G = 4^n, applied block-diagonally to every contiguous group of G input
  features, giving an orthogonal symmetric R; weights stored as W R and
  activations rotated as X R at run time.
* same page, section "Weight quantization": one scale per output row equal to
  the row's largest magnitude over 127, codes rounded and clamped to
  [-127, 127].
* same page, section "Runtime activation quantization": the same rule per
  activation row (one dynamic scale over the whole rotated row), the signed
  32-bit integer accumulation A = Qx Qw^T, and Y ~= A s_x[r] s_w[o] + b[o].
* "Add experimental W8A8 MatMul with optional QuaRot-style rotation"
  (gemma.cpp issue), section "Rotation method": the randomized block variant,
  in its stated order -- a fixed +-1 diagonal, then a Walsh-Hadamard
  transform, then scaling by 1/sqrt(block) -- applied identically to
  activation rows and to transposed-weight rows.
* sglang PR 34581 summary page, section on implementation
  (kitchen_int8 layer routing): layers whose input width is not a multiple of
  the group size stay on the unquantised BF16 linear.
* stable-diffusion.cpp PR "load ConvRot int4 and per-channel int8
  safetensors", sections "Solution" and "The rotation": int4 weights are the
  rotated weight quantised to [-7, 7] with one scale per output channel,
  adjacent code pairs packed into one byte (W4A8 here: the int8 activation
  codes against those weight codes, same accumulation and epilogue).
* "Add experimental W8A8 MatMul ..." (gemma.cpp issue), the maintainer's
  review comment: data-free smoothing scales of an FFN's intermediate
  channels (L2 or max norms), applied to the weights before the rotation.
* "INT8 Convrot Safetensors", LoRA paragraph: the runtime adapter
  correction computed from the unrotated activation and added to the base
  output.

Readings taken where the pages are silent (all listed in the design notes of
the repository):

* ``round`` is round-half-to-even (``np.rint``).
* ``X_rot / s`` is an IEEE fp32 division of the fp32 rotated value by the fp32
  scale, and the scale is an IEEE fp32 division of the fp32 row maximum by 127.
* The rotation is evaluated in fp64 from the exact upcast of the fp32 or bf16
  input and then rounded once to fp32.
* An all-zero row has scale 0 and all-zero codes.
* Walsh-Hadamard order for the randomized variant is the natural (Sylvester)
  order H[i, j] = (-1)^popcount(i & j); the sign vector is an explicit input
  of length K (one sign per input feature).
* Y is evaluated in fp64 and rounded once to fp32; bf16 outputs are the
  round-half-to-even bf16 of that fp32 value.

Pins (tests/test_oracle.py, CPU-only) tie every function here to something
other than itself: the printed H4, exact orthogonality/symmetry, the base-4
digit closed form, scipy's Sylvester matrix, rotation invariance in fp64,
Parseval, a one-hot worked example whose output is known in closed form,
brute-force integer loops, and torch's bf16 rounding; for int4, the page's
code range, exact-tie rounding, a hand-packed nibble example, every byte
decoded, and the page's correlation check of rotated against un-rotated
weights; for smoothing, closed forms on scaled unit rows, the norms after
scaling, the zero-norm rule and the gated FFN's invariance; for LoRA, the
merged-weight identity on values that bf16 holds exactly, a one-hot closed
form, the bf16 rounding of the intermediate and a brute-force loop.
Nothing here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

REGULAR = "regular"
RANDOMIZED = "randomized"

QMAX = 127


# ---------------------------------------------------------------------------
# Rotation matrices
# ---------------------------------------------------------------------------

def h4() -> np.ndarray:
    """The 4x4 normalised regular Hadamard matrix H4 (fp64).

    "INT8 Convrot Safetensors", "How INT8 convrot works": the printed integer
    matrix divided by 2.  Every row sums to 1 and R is its own inverse.
    """
    m = np.array(
        [[1, 1, 1, -1],
         [1, 1, -1, 1],
         [1, -1, 1, 1],
         [-1, 1, 1, 1]],
        dtype=np.float64,
    )
    return m / 2.0


def _log4(G: int) -> int:
    n = 0
    g = G
    while g > 1 and g % 4 == 0:
        g //= 4
        n += 1
    if g != 1 or G < 4:
        raise ValueError(f"regular ConvRot group size must be a power of 4 >= 4, got {G}")
    return n


def regular_rotation(G: int) -> np.ndarray:
    """R_G = H4 (x) H4 (x) ... (n factors) for G = 4^n, fp64 (entries +-2^-n).

    "INT8 Convrot Safetensors", "How INT8 convrot works": the normalised
    Kronecker power of H4.  All factors are equal, so the factor order is
    immaterial.
    """
    n = _log4(G)
    r = np.ones((1, 1), dtype=np.float64)
    for _ in range(n):
        r = np.kron(r, h4())
    return r


def sylvester(G: int) -> np.ndarray:
    """Unnormalised Walsh-Hadamard matrix of order G = 2^m in natural order.

    H[i, j] = (-1)^popcount(i & j).  Built by the doubling recursion
    [[H, H], [H, -H]].
    """
    if G < 1 or (G & (G - 1)) != 0:
        raise ValueError(f"Walsh-Hadamard order must be a power of 2, got {G}")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < G:
        h = np.block([[h, h], [h, -h]])
    return h


def randomized_block(G: int, d: np.ndarray) -> np.ndarray:
    """Dense form T = (1/sqrt G) H D of the randomized block transform.

    "Add experimental W8A8 MatMul ...", "Rotation method": signs first, then
    the Walsh-Hadamard transform, then 1/sqrt(G).  T acts on a column vector
    v as t(v) = T v; it is orthonormal but not symmetric.
    """
    d = np.asarray(d, dtype=np.float64).reshape(G)
    if not np.all(np.abs(d) == 1.0):
        raise ValueError("Rademacher signs must be +-1")
    return sylvester(G) @ np.diag(d) / np.sqrt(G)


# ---------------------------------------------------------------------------
# Rotation of rows
# ---------------------------------------------------------------------------

def _check_rows(X: np.ndarray, G: int) -> np.ndarray:
    X = np.asarray(X)
    if X.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    if X.shape[1] % G != 0:
        raise ValueError(f"K={X.shape[1]} is not a multiple of G={G}")
    X64 = X.astype(np.float64)
    if not np.all(np.isfinite(X64)):
        raise ValueError("non-finite input is outside the method's domain")
    return X64


def rotate64(X: np.ndarray, G: int, kind: str = REGULAR,
             signs: np.ndarray | None = None) -> np.ndarray:
    """Group-wise rotation of every row of X, evaluated in fp64.

    REGULAR:    each contiguous G-column block x_b of a row becomes x_b R_G
                ("How INT8 convrot works": X_rot = X R with block-diagonal R).
    RANDOMIZED: each block becomes t(x_b) = (1/sqrt G) H (d_b * x_b), the
                signs d_b being the block's slice of the length-K sign vector
                ("Rotation method").  Written for a row vector: first the
                elementwise signs, then the Walsh-Hadamard transform (H is
                symmetric, so x H = (H x^T)^T), then the 1/sqrt(G) factor.
    """
    X64 = _check_rows(X, G)
    rows, K = X64.shape
    nb = K // G
    blocks = X64.reshape(rows, nb, G)
    if kind == REGULAR:
        if signs is not None:
            raise ValueError("signs are only used by the randomized rotation")
        out = blocks @ regular_rotation(G)
    elif kind == RANDOMIZED:
        if signs is None:
            raise ValueError("the randomized rotation needs a sign vector")
        d = np.asarray(signs).astype(np.float64).reshape(nb, G)
        if not np.all(np.abs(d) == 1.0):
            raise ValueError("Rademacher signs must be +-1")
        signed = blocks * d[None, :, :]
        out = (signed @ sylvester(G)) / np.sqrt(G)
    else:
        raise ValueError(f"unknown rotation kind {kind!r}")
    return out.reshape(rows, K)


def rotate(X: np.ndarray, G: int, kind: str = REGULAR,
           signs: np.ndarray | None = None) -> np.ndarray:
    """fp32 rotated rows: the fp64 rotation rounded once to fp32."""
    return rotate64(X, G, kind, signs).astype(np.float32)


# ---------------------------------------------------------------------------
# Per-row symmetric int8 quantisation
# ---------------------------------------------------------------------------

def quantize_rows(Xr32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row absmax int8 quantisation of fp32 rows.

    "Weight quantization" / "Runtime activation quantization":
        s[r]    = max_i |x[r, i]| / 127            (fp32 IEEE division)
        q[r, i] = clamp(round(x[r, i] / s[r]), -127, 127)
    with round = half-to-even and the division in fp32.  A row whose maximum
    is 0 gets s = 0 and q = 0.
    Returns (q int8 [rows, K], s fp32 [rows]).
    """
    x = np.asarray(Xr32)
    if x.dtype != np.float32:
        raise TypeError("quantize_rows expects the fp32 rotated rows")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (amax / np.float32(QMAX)).astype(np.float32)
    q = np.zeros(x.shape, dtype=np.int8)
    nz = s > 0
    if np.any(nz):
        v = (x[nz] / s[nz][:, None]).astype(np.float32)
        q[nz] = np.clip(np.rint(v), -QMAX, QMAX).astype(np.int8)
    return q, s


def code_values(Xr32: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The fp32 pre-rounding code values v = x / s (0 for zero rows).

    Exposed so that parity checks can decide whether an element sits next to
    a rounding tie.
    """
    x = np.asarray(Xr32, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    v = np.zeros(x.shape, dtype=np.float32)
    nz = s > 0
    v[nz] = (x[nz] / s[nz][:, None]).astype(np.float32)
    return v


def group_absmax(Xr32: np.ndarray, G: int) -> np.ndarray:
    """Largest magnitude of every contiguous G-group of fp32 rotated rows,
    [rows, K / G].

    Producer fusion of the next layer's rotation and row maximum (the
    "Backend support" section of "INT8 Convrot Safetensors" names the
    rotation, the row-wise maximum reduction and the quantisation as the
    fused activation-side work): a producing layer can emit these per-group
    maxima of its rotated output, and the whole-row maximum that sets the
    scale in "Runtime activation quantization" is their maximum, because the
    groups partition the row.  Zero groups give 0.
    """
    x = np.asarray(Xr32)
    if x.dtype != np.float32:
        raise TypeError("group_absmax expects the fp32 rotated rows")
    rows, K = x.shape
    if K % G:
        raise ValueError("K must be a multiple of G")
    return np.max(np.abs(x).reshape(rows, K // G, G), axis=2) if K else np.zeros((rows, 0), np.float32)


def pack(X: np.ndarray, G: int, kind: str = REGULAR,
         signs: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rotate then quantise rows (activations at run time, weights offline).

    Returns (q int8, s fp32, rotated fp32 rows).
    """
    xr = rotate(X, G, kind, signs)
    q, s = quantize_rows(xr)
    return q, s, xr


# ---------------------------------------------------------------------------
# int4 weights (W4A8)
# ---------------------------------------------------------------------------
#
# stable-diffusion.cpp PR "load ConvRot int4 and per-channel int8
# safetensors", sections "Solution" and "The rotation": ConvRot int4 weights
# are the rotated weight W R quantised to integers in [-7, 7] with one scale
# per output channel, and the payload packs adjacent pairs of codes into one
# byte.  Readings taken where the page is silent:
#   * the int4 rule is the int8 rule with 7 in place of 127:
#     s = max |x| / 7 (fp32 division), q = clamp(round_half_even(x / s), -7, 7);
#   * a byte holds element 2j in its low nibble and element 2j + 1 in its high
#     nibble, each as a 4-bit two's complement value (the page's "+8 bias
#     lands inside Q4_0's nibble range" implies signed nibbles).

QMAX4 = 7


def quantize_rows_int4(Xr32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row absmax int4 quantisation of fp32 rows.

        s[r]    = max_i |x[r, i]| / 7              (fp32 IEEE division)
        q[r, i] = clamp(round(x[r, i] / s[r]), -7, 7)
    round = half-to-even, the division in fp32; an all-zero row gets s = 0 and
    q = 0.  Returns (q int8 [rows, K] with values in [-7, 7], s fp32 [rows]).
    """
    x = np.asarray(Xr32)
    if x.dtype != np.float32:
        raise TypeError("quantize_rows_int4 expects the fp32 rotated rows")
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (amax / np.float32(QMAX4)).astype(np.float32)
    q = np.zeros(x.shape, dtype=np.int8)
    nz = s > 0
    if np.any(nz):
        v = (x[nz] / s[nz][:, None]).astype(np.float32)
        q[nz] = np.clip(np.rint(v), -QMAX4, QMAX4).astype(np.int8)
    return q, s


def pack_nibbles(q4: np.ndarray) -> np.ndarray:
    """Pack int4 codes [rows, K] (K even) into bytes [rows, K / 2]: byte j holds
    code 2j in its low nibble and code 2j + 1 in its high nibble, each as 4-bit
    two's complement."""
    q = np.asarray(q4)
    if q.dtype != np.int8 or q.ndim != 2 or q.shape[1] % 2:
        raise ValueError("pack_nibbles expects int8 codes [rows, even K]")
    if np.any(q < -8) or np.any(q > 7):
        raise ValueError("codes outside the 4-bit range")
    u = q.astype(np.int16) & 0xF
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: bytes [rows, K / 2] -> int8 codes [rows, K]."""
    b = np.asarray(b)
    if b.dtype != np.uint8 or b.ndim != 2:
        raise ValueError("unpack_nibbles expects uint8 [rows, bytes]")
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    q = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def pack_weight_int4(W: np.ndarray, G: int, kind: str = REGULAR,
                     signs: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Offline int4 weight: rotate, quantise to [-7, 7] per output row, pack
    nibble pairs.  Returns (bytes uint8 [N, K / 2], s fp32 [N], codes int8,
    rotated fp32 rows).  A W4A8 linear is then int_gemm(Qx,
    unpack_nibbles(bytes)) followed by the same epilogue as the int8 weight."""
    wr = rotate(W, G, kind, signs)
    q, s = quantize_rows_int4(wr)
    return pack_nibbles(q), s, q, wr


# ---------------------------------------------------------------------------
# Data-free smoothing of an FFN's intermediate channels
# ---------------------------------------------------------------------------
#
# "Add experimental W8A8 MatMul with optional QuaRot-style rotation"
# (gemma.cpp issue), maintainer's review comment: scale the weights before
# the rotation without calibration data -- max norms as in SmoothQuant and
# DuQuant++, or the square root of the ratio of the W_up to W_down L2 column
# norms -- so the quantisation range shrinks, the factor being pulled into the
# per-row scales.  Readings taken where the comment is silent:
#   * the scaled channel j is an intermediate channel of the FFN: row j of
#     W_up [F, K] and column j of W_down [K_out, F];
#   * s_j = sqrt(n_up[j] / n_down[j]) with n the L2 norm ("l2") or the largest
#     magnitude ("max"); W_up row j is divided by s_j and W_down column j
#     multiplied by it, which leaves both with norm sqrt(n_up n_down) and the
#     layer unchanged wherever up enters the intermediate linearly (the gated
#     FFN h = act(gate) * up);
#   * s_j = 1 where either norm is 0;
#   * s is computed in fp64 and stored as fp32; the scaled weights are the
#     fp64 quotient / product with that fp32 s, rounded once to fp32.


def smoothing_scales(W_up: np.ndarray, W_down: np.ndarray, norm: str = "l2") -> np.ndarray:
    """Per-channel smoothing scales s [F] (fp32) of an FFN with W_up [F, K]
    and W_down [K_out, F]."""
    up = np.asarray(W_up, np.float64)
    dn = np.asarray(W_down, np.float64)
    if up.ndim != 2 or dn.ndim != 2 or dn.shape[1] != up.shape[0]:
        raise ValueError("W_up [F, K] and W_down [K_out, F] expected")
    if norm == "l2":
        n_up = np.sqrt(np.sum(up * up, axis=1))
        n_dn = np.sqrt(np.sum(dn * dn, axis=0))
    elif norm == "max":
        n_up = np.max(np.abs(up), axis=1)
        n_dn = np.max(np.abs(dn), axis=0)
    else:
        raise ValueError(f"unknown norm {norm!r}")
    ok = (n_up > 0) & (n_dn > 0)
    s = np.ones(up.shape[0], np.float64)
    s[ok] = np.sqrt(n_up[ok] / n_dn[ok])
    return s.astype(np.float32)


def apply_smoothing(W_up: np.ndarray, W_down: np.ndarray, s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(W_up / s per row, W_down * s per column), fp64 then rounded once to fp32."""
    s64 = np.asarray(s, np.float32).astype(np.float64)
    up = (np.asarray(W_up, np.float64) / s64[:, None]).astype(np.float32)
    dn = (np.asarray(W_down, np.float64) * s64[None, :]).astype(np.float32)
    return up, dn


# ---------------------------------------------------------------------------
# Runtime LoRA correction from the unrotated activation
# ---------------------------------------------------------------------------
#
# "INT8 Convrot Safetensors", LoRA paragraph: adapters are applied at run
# time without touching the int8 weights; the convrot path computes the base
# output and the adapter computes its correction from the original,
# unrotated activation and adds it to that output.  Readings taken where the
# page is silent:
#   * the adapter is the low-rank pair A [r, K] (down) and B [N, r] (up) with
#     a scalar scale (alpha / r):  dY = scale (X A^T) B^T;
#   * the rank-r intermediate T = X A^T is held in bf16 (the adapter's own
#     precision), the product T B^T accumulates in fp32 and scale multiplies
#     the sum; the correction is added to the base output in the output's
#     precision (fp32, or the sum rounded to bf16).


def lora_intermediate(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """T = X A^T in fp64, rounded once to bf16 (returned as fp32 values)."""
    T = np.asarray(X, np.float64) @ np.asarray(A, np.float64).T
    return bf16_round(T.astype(np.float32)) if T.size else T.astype(np.float32)


def lora_delta64(X: np.ndarray, A: np.ndarray, B: np.ndarray, scale: float) -> np.ndarray:
    """dY = scale (bf16(X A^T)) B^T in fp64."""
    T = lora_intermediate(X, A).astype(np.float64)
    return float(np.float32(scale)) * (T @ np.asarray(B, np.float64).T)


# ---------------------------------------------------------------------------
# Integer accumulation, epilogue, rounding
# ---------------------------------------------------------------------------

def int_gemm(Qx: np.ndarray, Qw: np.ndarray) -> np.ndarray:
    """A[r, o] = sum_i Qx[r, i] Qw[o, i] exactly, as int64.

    ("Runtime activation quantization": signed 32-bit accumulation.)  The
    product is formed by an fp64 BLAS matmul of the int8-valued matrices,
    which is exact: every partial sum is an integer of magnitude at most
    K * 127^2, far below 2^53.  The result is checked to fit in int32.
    """
    Qx = np.asarray(Qx)
    Qw = np.asarray(Qw)
    if Qx.dtype != np.int8 or Qw.dtype != np.int8:
        raise TypeError("int_gemm expects int8 codes")
    K = Qx.shape[1]
    if Qw.shape[1] != K:
        raise ValueError("inner dimensions differ")
    if K * QMAX * QMAX >= 2 ** 53:
        raise ValueError("K too large for exact fp64 accumulation")
    A = (Qx.astype(np.float64) @ Qw.astype(np.float64).T).astype(np.int64)
    if A.size and np.max(np.abs(A)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    return A


def int_gemm_bruteforce(Qx: np.ndarray, Qw: np.ndarray) -> np.ndarray:
    """Triple loop over Python integers (tiny shapes only)."""
    M, K = Qx.shape
    N = Qw.shape[0]
    A = np.zeros((M, N), dtype=np.int64)
    for r in range(M):
        for o in range(N):
            acc = 0
            for i in range(K):
                acc += int(Qx[r, i]) * int(Qw[o, i])
            A[r, o] = acc
    return A


def epilogue64(A: np.ndarray, s_x: np.ndarray, s_w: np.ndarray,
               bias: np.ndarray | None = None) -> np.ndarray:
    """Y[r, o] = A[r, o] * s_x[r] * s_w[o] + b[o], evaluated in fp64.

    ("Runtime activation quantization": the floating-point reconstruction.)
    """
    Y = np.asarray(A, dtype=np.float64) * np.asarray(s_x, np.float64)[:, None]
    Y = Y * np.asarray(s_w, np.float64)[None, :]
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even).

    Returns the bf16 values as fp32 (the low 16 bits cleared).  bf16 keeps the
    top 16 bits of the fp32 encoding; rounding adds half of the dropped range
    minus one, plus the lowest kept bit, before truncating.
    """
    x = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round expects finite input")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def linear(X: np.ndarray, Wq: np.ndarray, s_w: np.ndarray,
           bias: np.ndarray | None, G: int, kind: str = REGULAR,
           signs: np.ndarray | None = None) -> dict:
    """The full quantised linear for activations X against a packed weight.

    Returns a dict with the packed activation (q, s, rotated fp32), the exact
    accumulator A and the fp64 / fp32 outputs.
    """
    qx, sx, xr = pack(X, G, kind, signs)
    A = int_gemm(qx, Wq)
    y64 = epilogue64(A, sx, s_w, bias)
    return {"qx": qx, "sx": sx, "xrot": xr, "A": A, "y64": y64,
            "y32": y64.astype(np.float32)}


def linear_unquantized64(X: np.ndarray, W: np.ndarray,
                         bias: np.ndarray | None = None) -> np.ndarray:
    """Y = X W^T + b in fp64: the unquantised layer and the routed fallback.

    (sglang summary page, implementation section: layers whose input width
    is not divisible by the group size keep the plain BF16 linear.)
    """
    Y = np.asarray(X, np.float64) @ np.asarray(W, np.float64).T
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y


def routes_to_fallback(K: int, G: int) -> bool:
    """True when the layer must stay on the unquantised linear (K % G != 0)."""
    return K % G != 0
