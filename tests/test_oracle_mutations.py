"""Plant plausible mistakes into the oracle (CPU only) and check that the
pins catch every one of them."""

import numpy as np
import pytest

import oracle.convrot_oracle as O
from tests import oracle_pins as P

_h4 = O.h4
_sylvester = O.sylvester
_rotate64 = O.rotate64
_quantize_rows = O.quantize_rows
_epilogue64 = O.epilogue64
_int_gemm = O.int_gemm
_bf16_round = O.bf16_round
_randomized_block = O.randomized_block
_code_values = O.code_values
_group_absmax = O.group_absmax


def _h4_sign_flip():
    m = _h4().copy()
    m[0, 3] = -m[0, 3]
    return m


def _h4_unnormalised():
    return _h4() * 2.0


def _h4_wrong_row_order():
    return _h4()[::-1].copy()


def _rotate_strided_groups(X, G, kind=O.REGULAR, signs=None):
    # groups taken as columns {b, b + nb, ...} instead of contiguous blocks
    X = np.asarray(X, np.float64)
    rows, K = X.shape
    nb = K // G
    Xt = X.reshape(rows, G, nb).transpose(0, 2, 1).reshape(rows, K)
    out = _rotate64(Xt, G, kind, signs)
    return out.reshape(rows, nb, G).transpose(0, 2, 1).reshape(rows, K)


def _rotate_signs_after(X, G, kind=O.REGULAR, signs=None):
    if kind != O.RANDOMIZED:
        return _rotate64(X, G, kind, signs)
    X = np.asarray(X, np.float64)
    rows, K = X.shape
    nb = K // G
    d = np.asarray(signs, np.float64).reshape(nb, G)
    out = (X.reshape(rows, nb, G) @ O.sylvester(G)) * d[None] / np.sqrt(G)
    return out.reshape(rows, K)


def _rotate_no_normalise(X, G, kind=O.REGULAR, signs=None):
    out = _rotate64(X, G, kind, signs)
    return out * np.sqrt(G) if kind == O.RANDOMIZED else out


def _quant_128(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(128)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(x[nz] / s[nz][:, None]), -127, 127).astype(np.int8)
    return q, s


def _quant_half_away(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(127)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    v = (x[nz] / s[nz][:, None]).astype(np.float32)
    q[nz] = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8)
    return q, s


def _quant_truncate(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(127)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    q[nz] = np.clip(np.trunc(x[nz] / s[nz][:, None]), -127, 127).astype(np.int8)
    return q, s


def _quant_first_group_scale(x):
    # scale from the first 4 columns only instead of the whole row
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x[:, :4]), axis=1)
    s = (amax / np.float32(127)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(x[nz] / s[nz][:, None]), -127, 127).astype(np.int8)
    return q, s


def _epi_no_bias(A, sx, sw, bias=None):
    return _epilogue64(A, sx, sw, None)


def _epi_no_sw(A, sx, sw, bias=None):
    return _epilogue64(A, sx, np.ones_like(np.asarray(sw)), bias)


def _epi_swapped(A, sx, sw, bias=None):
    A = np.asarray(A, np.float64)
    Y = A * np.resize(np.asarray(sw, np.float64), A.shape[0])[:, None]
    Y = Y * np.resize(np.asarray(sx, np.float64), A.shape[1])[None, :]
    return Y + (0 if bias is None else np.asarray(bias, np.float64)[None, :])


def _gemm_untransposed(Qx, Qw):
    return (Qx.astype(np.float64) @ Qw.astype(np.float64).T[::-1]).astype(np.int64) \
        if Qx.shape[1] == Qw.shape[1] else None


def _gemm_float32(Qx, Qw):
    return (Qx.astype(np.float32) @ Qw.astype(np.float32).T).astype(np.int64)


def _bf16_truncate(x):
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def _sylvester_wrong_sign(G):
    h = _sylvester(G).copy()
    h[-1, -1] = -h[-1, -1]
    return h



_quantize_rows_int4 = O.quantize_rows_int4
_pack_nibbles = O.pack_nibbles
_unpack_nibbles = O.unpack_nibbles


def _quant4_divides_by_8(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(8)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    q[nz] = np.clip(np.rint(x[nz] / s[nz][:, None]), -7, 7).astype(np.int8)
    return q, s


def _quant4_half_away(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(7)).astype(np.float32)
    q = np.zeros(x.shape, np.int8)
    nz = s > 0
    v = x[nz] / s[nz][:, None]
    q[nz] = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -7, 7).astype(np.int8)
    return q, s


def _nibbles_high_first(q4):
    u = np.asarray(q4).astype(np.int16) & 0xF
    return ((u[:, 0::2] << 4) | u[:, 1::2]).astype(np.uint8)


def _unpack_unsigned(b):
    q = np.empty((b.shape[0], 2 * b.shape[1]), np.int16)
    q[:, 0::2] = b & 0xF
    q[:, 1::2] = b >> 4
    return q.astype(np.int8)


def _unpack_swapped(b):
    q = _unpack_nibbles(b)
    out = q.copy()
    out[:, 0::2], out[:, 1::2] = q[:, 1::2], q[:, 0::2]
    return out



_smoothing_scales = O.smoothing_scales
_apply_smoothing = O.apply_smoothing


def _smooth_inverted_ratio(W_up, W_down, norm="l2"):
    s = _smoothing_scales(W_up, W_down, norm)
    return (1.0 / s).astype(np.float32)


def _smooth_no_sqrt(W_up, W_down, norm="l2"):
    s = _smoothing_scales(W_up, W_down, norm).astype(np.float64)
    return (s * s).astype(np.float32)


def _smooth_applied_backwards(W_up, W_down, s):
    s64 = np.asarray(s, np.float64)
    return ((np.asarray(W_up, np.float64) * s64[:, None]).astype(np.float32),
            (np.asarray(W_down, np.float64) / s64[None, :]).astype(np.float32))


def _smooth_rows_of_down(W_up, W_down, norm="l2"):
    # norms of W_down's rows instead of its columns (only shapes with K_out == F survive)
    up = np.asarray(W_up, np.float64)
    dn = np.asarray(W_down, np.float64)
    n_up = np.sqrt(np.sum(up * up, axis=1)) if norm == "l2" else np.max(np.abs(up), axis=1)
    n_dn = np.sqrt(np.sum(dn * dn, axis=1)) if norm == "l2" else np.max(np.abs(dn), axis=1)
    n_dn = np.resize(n_dn, n_up.shape)
    return np.sqrt(np.where(n_dn > 0, n_up / np.where(n_dn > 0, n_dn, 1), 1)).astype(np.float32)



_lora_intermediate = O.lora_intermediate
_lora_delta64 = O.lora_delta64


def _lora_no_bf16(X, A):
    return (np.asarray(X, np.float64) @ np.asarray(A, np.float64).T).astype(np.float32)


def _lora_up_read_as_rn(X, A, B, scale):
    # B [N, r] read as if it were stored [r, N] row-major (a layout mistake)
    T = _lora_intermediate(X, A).astype(np.float64)
    Bw = np.asarray(B, np.float64)
    Bs = Bw.ravel().reshape(Bw.shape[1], Bw.shape[0]).T
    return float(scale) * (T @ Bs.T)


def _lora_no_scale(X, A, B, scale):
    return _lora_delta64(X, A, B, 1.0)


def _code_values_fp64(x, s):
    # the quotient left in fp64 instead of rounded to fp32
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    v = np.zeros(x.shape)
    nz = s > 0
    v[nz] = x[nz] / s[nz][:, None]
    return v


def _code_values_reciprocal(x, s):
    # x * (127 / amax) in fp32 instead of the division x / s
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)
    inv = np.zeros_like(amax)
    nz = amax > 0
    inv[nz] = (np.float32(127) / amax[nz]).astype(np.float32)
    return (x * inv[:, None]).astype(np.float32)


def _code_values_unmasked(x, s):
    # zero rows divided by a zero scale (NaN codes) instead of v = 0
    x = np.asarray(x, np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (x / np.asarray(s, np.float32)[:, None]).astype(np.float32)


def _group_absmax_strided(x, G):
    # groups taken as strided columns instead of contiguous blocks
    x = np.asarray(x, np.float32)
    rows, K = x.shape
    return np.max(np.abs(x).reshape(rows, G, K // G), axis=1)


def _group_absmax_signed(x, G):
    # the largest value instead of the largest magnitude
    x = np.asarray(x, np.float32)
    rows, K = x.shape
    return np.max(x.reshape(rows, K // G, G), axis=2)


MUTATIONS = {
    "h4_sign_flip": ("h4", _h4_sign_flip),
    "h4_unnormalised": ("h4", _h4_unnormalised),
    "h4_row_order": ("h4", _h4_wrong_row_order),
    "rotate_strided_groups": ("rotate64", _rotate_strided_groups),
    "randomized_signs_after_wht": ("rotate64", _rotate_signs_after),
    "randomized_no_normalise": ("rotate64", _rotate_no_normalise),
    "sylvester_wrong_sign": ("sylvester", _sylvester_wrong_sign),
    "quant_divides_by_128": ("quantize_rows", _quant_128),
    "quant_half_away": ("quantize_rows", _quant_half_away),
    "quant_truncates": ("quantize_rows", _quant_truncate),
    "quant_partial_row_scale": ("quantize_rows", _quant_first_group_scale),
    "code_values_fp64": ("code_values", _code_values_fp64),
    "code_values_reciprocal": ("code_values", _code_values_reciprocal),
    "code_values_zero_rows_nan": ("code_values", _code_values_unmasked),
    "group_absmax_strided_groups": ("group_absmax", _group_absmax_strided),
    "group_absmax_signed": ("group_absmax", _group_absmax_signed),
    "epilogue_drops_bias": ("epilogue64", _epi_no_bias),
    "epilogue_drops_weight_scale": ("epilogue64", _epi_no_sw),
    "epilogue_swaps_scales": ("epilogue64", _epi_swapped),
    "gemm_wrong_operand_order": ("int_gemm", _gemm_untransposed),
    "gemm_float32_accumulation": ("int_gemm", _gemm_float32),
    "bf16_truncates": ("bf16_round", _bf16_truncate),
    "quant4_divides_by_8": ("quantize_rows_int4", _quant4_divides_by_8),
    "quant4_half_away": ("quantize_rows_int4", _quant4_half_away),
    "nibbles_high_first": ("pack_nibbles", _nibbles_high_first),
    "unpack_without_sign": ("unpack_nibbles", _unpack_unsigned),
    "unpack_swapped_nibbles": ("unpack_nibbles", _unpack_swapped),
    "smooth_inverted_ratio": ("smoothing_scales", _smooth_inverted_ratio),
    "smooth_no_sqrt": ("smoothing_scales", _smooth_no_sqrt),
    "smooth_rows_of_down": ("smoothing_scales", _smooth_rows_of_down),
    "smooth_applied_backwards": ("apply_smoothing", _smooth_applied_backwards),
    "lora_intermediate_not_rounded": ("lora_intermediate", _lora_no_bf16),
    "lora_up_read_as_rn": ("lora_delta64", _lora_up_read_as_rn),
    "lora_scale_dropped": ("lora_delta64", _lora_no_scale),
}


def test_unmutated_oracle_passes_every_pin():
    assert P.run_all() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = P.run_all()
    assert failed, f"planted mistake {name!r} passed every pin"
