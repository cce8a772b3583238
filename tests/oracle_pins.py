"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
what the pages print, with a closed form, an invariant, a textbook routine or
brute force.  ``test_oracle.py`` runs them against the oracle as written, and
``test_oracle_mutations.py`` plants plausible mistakes into the oracle (on the
CPU, via monkeypatch) and asserts that at least one check catches each.
"""

from __future__ import annotations

import functools
import json
import os

import numpy as np
import scipy.linalg
import torch

import oracle.convrot_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
REGULAR_GS = (4, 16, 64, 256, 1024)


def load_printed_h4() -> np.ndarray:
    rows, div = [], None
    with open(os.path.join(GOLDEN, "h4_printed.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("divisor"):
                div = float(line.split()[1])
            else:
                rows.append([float(t) for t in line.split()])
    return np.array(rows) / div


def page_constants() -> dict:
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        return json.load(f)


def _digits4(i: int, n: int):
    return [(i >> (2 * k)) & 3 for k in range(n)]


@functools.lru_cache(maxsize=None)
def _closed_form_cached(G: int) -> np.ndarray:
    """R_G[i, j] = 2^-n * (-1)^{#{k : i_k + j_k = 3}} over base-4 digits.

    Follows from H4 = J/2 - (anti-diagonal): an entry of H4 is -1/2 exactly
    when its two indices add up to 3.
    """
    n = int(round(np.log(G) / np.log(4)))
    R = np.empty((G, G))
    for i in range(G):
        di = _digits4(i, n)
        for j in range(G):
            dj = _digits4(j, n)
            neg = sum(1 for a, b in zip(di, dj) if a + b == 3)
            R[i, j] = (-1.0) ** neg * 2.0 ** (-n)
    R.setflags(write=False)
    return R


def closed_form_regular(G: int) -> np.ndarray:
    return _closed_form_cached(G).copy()


# -- rotation matrices -------------------------------------------------------

def check_r4_printed():
    assert np.array_equal(O.regular_rotation(4), load_printed_h4())
    assert np.array_equal(O.h4(), load_printed_h4())


def check_regular_structure(G: int):
    R = O.regular_rotation(G)
    I = np.eye(G)
    assert R.shape == (G, G)
    assert np.array_equal(R @ R.T, I), "R R^T != I"
    assert np.array_equal(R, R.T), "R not symmetric"
    assert np.array_equal(R @ R, I), "R^2 != I"
    assert np.array_equal(R.sum(axis=1), np.ones(G)), "rows must sum to 1 (constant vector is fixed)"
    assert R.trace() == np.sqrt(G)


def check_regular_closed_form(G: int):
    assert np.array_equal(O.regular_rotation(G), closed_form_regular(G))


def check_sylvester(G: int):
    assert np.array_equal(O.sylvester(G), scipy.linalg.hadamard(G).astype(np.float64))


def check_randomized_orthonormal(G: int, seed: int = 0):
    d = np.where(np.random.default_rng(seed).integers(0, 2, G) == 0, 1.0, -1.0)
    T = O.randomized_block(G, d)
    assert np.max(np.abs(T @ T.T - np.eye(G))) <= 1e-15
    expected = scipy.linalg.hadamard(G) @ np.diag(d) / np.sqrt(G)
    assert np.max(np.abs(T - expected)) <= 1e-15


# -- rotation of rows ----------------------------------------------------------

def check_rotate_block_placement(G: int, K: int, seed: int = 1):
    """Explicit K x K block-diagonal matrix (scipy.linalg.block_diag)."""
    X = np.random.default_rng(seed).standard_normal((5, K))
    Rbig = scipy.linalg.block_diag(*([O.regular_rotation(G)] * (K // G)))
    assert np.max(np.abs(O.rotate64(X, G) - X @ Rbig)) <= 1e-12


def check_randomized_onehot_order(G: int, K: int, seed: int = 2):
    """t(e_j) = d_j * (column j of H) / sqrt(G): signs first, then WHT."""
    g = np.random.default_rng(seed)
    d = np.where(g.integers(0, 2, K) == 0, 1, -1).astype(np.int8)
    H = scipy.linalg.hadamard(G).astype(np.float64)
    for j in (0, 1, G - 1, G + 3, K - 1):
        if j >= K:
            continue
        x = np.zeros((1, K))
        x[0, j] = 1.0
        got = O.rotate64(x, G, O.RANDOMIZED, d)[0]
        b, jj = divmod(j, G)
        want = np.zeros(K)
        want[b * G:(b + 1) * G] = d[j] * H[:, jj] / np.sqrt(G)
        assert np.max(np.abs(got - want)) <= 1e-15


def check_invariance(G: int, kind: str, K: int, seed: int = 3):
    """X_rot W_rot^T == X W^T in fp64 within 1e-10 relative (Frobenius)."""
    g = np.random.default_rng(seed)
    X = g.standard_normal((7, K))
    W = g.standard_normal((9, K))
    signs = np.where(g.integers(0, 2, K) == 0, 1, -1).astype(np.int8) if kind == O.RANDOMIZED else None
    Xr = O.rotate64(X, G, kind, signs)
    Wr = O.rotate64(W, G, kind, signs)
    ref = X @ W.T
    err = np.linalg.norm(Xr @ Wr.T - ref) / np.linalg.norm(ref)
    assert err <= 1e-10, err


def check_parseval(G: int, kind: str, K: int, seed: int = 4):
    g = np.random.default_rng(seed)
    X = g.standard_normal((6, K)) * 3.0
    signs = np.where(g.integers(0, 2, K) == 0, 1, -1).astype(np.int8) if kind == O.RANDOMIZED else None
    Xr = O.rotate64(X, G, kind, signs)
    n0 = np.linalg.norm(X.reshape(6, K // G, G), axis=2)
    n1 = np.linalg.norm(Xr.reshape(6, K // G, G), axis=2)
    assert np.max(np.abs(n1 - n0) / n0) <= 1e-13


def check_onehot_spreading(G: int):
    """A row c*e_j rotates to +-c/sqrt(G) over j's group, 0 elsewhere; the
    codes are +-127 following the sign pattern of the closed form's row j."""
    n = int(round(np.log(G) / np.log(4)))
    K = 2 * G
    Rc = closed_form_regular(G)
    for j, c in ((0, 3.0), (G + 5 % G, -1.5), (K - 1, 0.75)):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, j] = c
        q, s, xr = O.pack(x, G)
        b, jj = divmod(j, G)
        want = np.zeros(K, dtype=np.float64)
        want[b * G:(b + 1) * G] = c * Rc[jj]
        assert np.array_equal(xr[0].astype(np.float64), want)
        mag = abs(c) * 2.0 ** (-n)
        assert s[0] == np.float32(np.float32(mag) / np.float32(127))
        qwant = np.zeros(K, dtype=np.int8)
        qwant[b * G:(b + 1) * G] = (127 * np.sign(c) * np.sign(Rc[jj])).astype(np.int8)
        assert np.array_equal(q[0], qwant)


def check_constant_row_fixed_point(G: int):
    x = np.full((1, 2 * G), 0.375, dtype=np.float32)
    q, s, xr = O.pack(x, G)
    assert np.array_equal(xr, x)
    assert np.all(q == 127)
    assert s[0] == np.float32(np.float32(0.375) / np.float32(127))


# -- quantisation ------------------------------------------------------------

def check_quant_invariants(seed: int = 5):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((16, 512)) * g.uniform(0.01, 100, (16, 1))).astype(np.float32)
    x[3] = 0.0
    x[7, 11] = 400.0
    q, s = O.quantize_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.min(q) >= -127 and np.max(q) <= 127
    for r in range(16):
        if r == 3:
            assert s[r] == 0 and np.all(q[r] == 0)
            continue
        amax = np.max(np.abs(x[r]))
        assert s[r] == np.float32(amax / np.float32(127))
        assert np.max(np.abs(q[r])) == 127
        assert abs(int(q[r, np.argmax(np.abs(x[r]))])) == 127
        err = np.abs(q[r].astype(np.float64) * float(s[r]) - x[r].astype(np.float64))
        assert np.max(err) <= 0.5 * float(s[r]) * (1 + 1e-4), "dequantisation error beyond half a step"


def check_quant_ties_half_even():
    # amax 127 gives s == 1 exactly, so the codes are rint of the values.
    x = np.array([[127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 126.5]], dtype=np.float32)
    q, s = O.quantize_rows(x)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 2, 4, -2, 0, 0, 2, 126]


def check_code_values(seed: int = 18):
    """``code_values`` is the value the quantiser rounds.  Rounded half to
    even and clamped it gives ``quantize_rows``' codes (int8) and
    ``quantize_rows_int4``' codes (int4), on rows of mixed magnitude, a
    zero row and a row with s = 1 and exact ties.  Each v is the correctly
    rounded fp32 quotient x / s: an fp64 division rounded once to fp32 is
    that quotient (53 >= 2 * 24 + 2 bits, so the double rounding is
    innocuous).  A zero row gives v = 0."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((12, 384)) * g.uniform(1e-3, 300, (12, 1))).astype(np.float32)
    x[2] = 0.0
    x[5, :8] = [127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 126.5]
    x[5, 8:] = np.clip(x[5, 8:], -100, 100)
    q, s = O.quantize_rows(x)
    v = O.code_values(x, s)
    assert v.dtype == np.float32 and v.shape == x.shape
    assert np.array_equal(np.clip(np.rint(v), -127, 127).astype(np.int8), q)
    assert s[5] == 1.0 and np.array_equal(v[5], x[5])
    assert np.all(v[2] == 0)
    nz = s > 0
    exact = (x[nz].astype(np.float64) / s[nz, None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(v[nz], exact)
    q4, s4 = O.quantize_rows_int4(x)
    v4 = O.code_values(x, s4)
    assert np.array_equal(np.clip(np.rint(v4), -7, 7).astype(np.int8), q4)
    assert np.all(v4[2] == 0)


def check_group_absmax(seed: int = 19):
    """The per-group maxima of a rotated row: their maximum is the row
    maximum that sets the scale (fp32(max / 127) equals quantize_rows' s);
    a one-hot row spreads over its own group only (|c| / sqrt(G) there, 0
    in every other group); brute force over the groups by a Python loop on
    a small case; zero rows give zeros."""
    g = np.random.default_rng(seed)
    for G in (4, 16, 64, 256):
        x = (g.standard_normal((6, 4 * G)) * g.uniform(0.1, 30, (6, 1))).astype(np.float32)
        x[4] = 0.0
        xr = O.rotate(x, G)
        pm = O.group_absmax(xr, G)
        assert pm.shape == (6, 4) and pm.dtype == np.float32
        _, s = O.quantize_rows(xr)
        assert np.array_equal((np.max(pm, axis=1) / np.float32(127)).astype(np.float32), s)
        assert np.all(pm[4] == 0)
        for r in (0, 5):
            for b in range(4):
                assert pm[r, b] == max(abs(float(v)) for v in xr[r, b * G:(b + 1) * G])
        one = np.zeros((1, 4 * G), np.float32)
        one[0, 2 * G + G - 1] = -3.0
        pm1 = O.group_absmax(O.rotate(one, G), G)
        assert pm1[0, 2] == np.float32(3.0 / np.sqrt(G)) and np.all(pm1[0, [0, 1, 3]] == 0)


def check_qmax_from_pages():
    consts = page_constants()
    assert O.QMAX == consts["qmax"]


# -- integer GEMM, epilogue, rounding -----------------------------------------

def check_int_gemm_bruteforce(seed: int = 6):
    g = np.random.default_rng(seed)
    for (M, N, K) in ((3, 5, 8), (4, 3, 32), (1, 7, 16)):
        Qx = g.integers(-127, 128, (M, K)).astype(np.int8)
        Qw = g.integers(-127, 128, (N, K)).astype(np.int8)
        Qx[0, 0], Qw[0, 0], Qx[-1, -1], Qw[-1, -1] = 127, -127, -127, -127
        assert np.array_equal(O.int_gemm(Qx, Qw), O.int_gemm_bruteforce(Qx, Qw))


def check_int_gemm_extremes():
    K = 12288
    Qx = np.full((2, K), 127, dtype=np.int8)
    Qw = np.full((3, K), -127, dtype=np.int8)
    Qw[1] = 127
    A = O.int_gemm(Qx, Qw)
    assert A[0, 0] == -K * 127 * 127 and A[1, 1] == K * 127 * 127


def check_int_gemm_large_random(seed: int = 10):
    """Large K against numpy's exact int64 matmul (no floating point)."""
    g = np.random.default_rng(seed)
    K = 12288
    Qx = g.integers(-127, 128, (6, K)).astype(np.int8)
    Qw = g.integers(-127, 128, (5, K)).astype(np.int8)
    Qx[:, :4096] = 127
    Qw[:, :4096] = 127
    want = Qx.astype(np.int64) @ Qw.astype(np.int64).T
    assert np.array_equal(O.int_gemm(Qx, Qw), want)


def check_epilogue_scalar(seed: int = 7):
    g = np.random.default_rng(seed)
    A = g.integers(-10 ** 6, 10 ** 6, (3, 4))
    sx = g.uniform(0.001, 1, 3).astype(np.float32)
    sw = g.uniform(0.001, 1, 4).astype(np.float32)
    b = g.standard_normal(4).astype(np.float32)
    Y = O.epilogue64(A, sx, sw, b)
    for r in range(3):
        for o in range(4):
            want = float(A[r, o]) * float(sx[r]) * float(sw[o]) + float(b[o])
            assert abs(Y[r, o] - want) <= 1e-12 * max(1.0, abs(want))
    Y0 = O.epilogue64(A, sx, sw, None)
    for r in range(3):
        for o in range(4):
            assert abs(Y0[r, o] - float(A[r, o]) * float(sx[r]) * float(sw[o])) <= 1e-12 * max(1.0, abs(Y0[r, o]))


def check_onehot_linear_closed_form(G: int):
    """X rows c_r e_{j_r}, W rows w_o e_{k_o}: the quantised linear returns
    X W^T + b (= c_r w_o [j_r == k_o] + b_o) up to fp32 scale rounding."""
    K = 2 * G
    js = [0, 5 % G, G + 1, K - 1]
    ks = [0, 5 % G, 1, G + 1, K - 1, G]
    cs = np.array([2.0, -0.5, 1.25, 4.0], dtype=np.float32)
    ws = np.array([0.03, -0.02, 0.5, 0.25, -1.0, 0.125], dtype=np.float32)
    X = np.zeros((len(js), K), dtype=np.float32)
    W = np.zeros((len(ks), K), dtype=np.float32)
    for r, (j, c) in enumerate(zip(js, cs)):
        X[r, j] = c
    for o, (k, w) in enumerate(zip(ks, ws)):
        W[o, k] = w
    b = np.linspace(-0.1, 0.1, len(ks)).astype(np.float32)
    qw, sw, _ = O.pack(W, G)
    out = O.linear(X, qw, sw, b, G)
    truth = X.astype(np.float64) @ W.astype(np.float64).T + b
    assert np.max(np.abs(out["y64"] - truth)) <= 1e-6 * np.max(np.abs(truth))
    # Exactly orthogonal patterns must cancel to an integer zero.
    for r, j in enumerate(js):
        for o, k in enumerate(ks):
            if j != k:
                assert out["A"][r, o] == 0
            else:
                assert abs(out["A"][r, o]) == 127 * 127 * G


def check_bf16_round(seed: int = 8):
    g = np.random.default_rng(seed)
    x = (g.standard_normal(20000) * 10.0 ** g.uniform(-8, 8, 20000)).astype(np.float32)
    # exact ties and near-ties
    base = x.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, (ties.view(np.uint32) + 1).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_round(x), want)


def check_fallback_bruteforce(seed: int = 9):
    g = np.random.default_rng(seed)
    X = g.standard_normal((3, 6))
    W = g.standard_normal((4, 6))
    b = g.standard_normal(4)
    Y = O.linear_unquantized64(X, W, b)
    for r in range(3):
        for o in range(4):
            want = sum(X[r, i] * W[o, i] for i in range(6)) + b[o]
            assert abs(Y[r, o] - want) <= 1e-12


def check_routing():
    consts = page_constants()
    G = consts["common_group_size"]
    assert O.routes_to_fallback(consts["routed_width"], G)
    for K in (1024, 3072, 6144, 12288):
        assert not O.routes_to_fallback(K, G)
    for K in (1152, 6912):
        assert O.routes_to_fallback(K, 1024)
        assert not O.routes_to_fallback(K, 64)
        assert not O.routes_to_fallback(K, consts["randomized_block"])



# -- int4 weights (W4A8) ------------------------------------------------------

def check_qmax4_from_pages():
    assert O.QMAX4 == page_constants()["qmax_int4"]


def check_int4_ties_half_even():
    # amax 7 gives s == 1 exactly, so the codes are rint of the values.
    x = np.array([[7.0, 2.5, 3.5, -2.5, 0.5, -1.5, 6.5, -0.5]], dtype=np.float32)
    q, s = O.quantize_rows_int4(x)
    assert s[0] == 1.0
    assert q[0].tolist() == [7, 2, 4, -2, 0, -2, 6, 0]


def check_int4_invariants(seed: int = 11):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((6, 96)) * g.uniform(0.01, 50, (6, 1))).astype(np.float32)
    x[2] = 0.0
    q, s = O.quantize_rows_int4(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[2] == 0 and not np.any(q[2])
    for r in (0, 1, 3, 4, 5):
        assert np.max(np.abs(q[r])) == 7
        assert abs(int(q[r, np.argmax(np.abs(x[r]))])) == 7
        assert s[r] == np.float32(np.max(np.abs(x[r])) / np.float32(7))
        err = np.abs(q[r].astype(np.float64) * float(s[r]) - x[r].astype(np.float64))
        assert np.max(err) <= 0.5 * float(s[r]) * (1 + 1e-4)


def check_nibble_worked_example():
    # By hand: byte j = (code 2j mod 16) + 16 (code 2j+1 mod 16).
    # (1, -1) -> 0x1 + 0xF0; (7, -7) -> 0x7 + 0x90; (0, 5) -> 0x50; (-3, 2) -> 0xD + 0x20
    q = np.array([[1, -1, 7, -7, 0, 5, -3, 2]], dtype=np.int8)
    b = O.pack_nibbles(q)
    assert b.dtype == np.uint8 and b.shape == (1, 4)
    assert b[0].tolist() == [0xF1, 0x97, 0x50, 0x2D]
    assert np.array_equal(O.unpack_nibbles(b), q)


def check_nibble_bytes_exhaustive():
    # Every byte decodes to (low, high) nibble as 4-bit two's complement:
    # a nibble n means n - 16 when its top bit is set.
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = O.unpack_nibbles(b)
    for v in range(256):
        lo = (v & 0xF) - 16 if v & 0x8 else v & 0xF
        hi = (v >> 4) - 16 if v & 0x80 else v >> 4
        assert (int(q[0, 2 * v]), int(q[0, 2 * v + 1])) == (lo, hi)
    codes = np.array([[a, c] for a in range(-7, 8) for c in range(-7, 8)], dtype=np.int8)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(codes)), codes)


def check_int4_rotation_correlation(seed: int = 12):
    """The PR's verification: dequantised int4 weights of W R correlate with
    W only once un-rotated by R (R is symmetric and orthogonal).  Read as-is
    the correlation is trace(R) / K = 2^-n for G = 4^n (1/16 at G = 256), the
    page's 0.06."""
    consts = page_constants()
    g = np.random.default_rng(seed)
    G = 256
    W = g.standard_normal((96, 2 * G)).astype(np.float32)
    b, s, q, _ = O.pack_weight_int4(W, G)
    deq = O.unpack_nibbles(b).astype(np.float64) * s[:, None].astype(np.float64)
    unrot = O.rotate64(deq, G)  # R is its own inverse
    corr = lambda a, c: float(np.corrcoef(a.ravel(), c.ravel())[0, 1])
    assert abs(corr(deq, W) - 1.0 / 16) < 0.03
    assert abs(corr(deq, W) - consts["int4_corr_as_is"]) < 0.03
    assert corr(unrot, W) >= consts["int4_corr_unrotated_min"]


def check_w4a8_int_gemm_bruteforce(seed: int = 13):
    g = np.random.default_rng(seed)
    Qx = g.integers(-127, 128, (3, 32)).astype(np.int8)
    Qw = g.integers(-7, 8, (5, 32)).astype(np.int8)
    A = O.int_gemm(Qx, O.unpack_nibbles(O.pack_nibbles(Qw)))
    assert np.array_equal(A, O.int_gemm_bruteforce(Qx, Qw))



# -- data-free smoothing (FFN intermediate channels) ---------------------------

def _unit_ffn(seed: int):
    """W_up row j = c_j u_j and W_down column j = d_j v_j with unit u, v (L2)."""
    g = np.random.default_rng(seed)
    F, K, Ko = 6, 32, 24
    u = g.standard_normal((F, K))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    v = g.standard_normal((Ko, F))
    v /= np.linalg.norm(v, axis=0, keepdims=True)
    c = np.array([1.0, 4.0, 0.25, 9.0, 2.0, 0.5])
    d = np.array([1.0, 1.0, 4.0, 0.01, 8.0, 0.5])
    return u * c[:, None], v * d[None, :], c, d


def check_smoothing_closed_form(seed: int = 14):
    up, dn, c, d = _unit_ffn(seed)
    s = O.smoothing_scales(up, dn, "l2")
    assert s.dtype == np.float32
    assert np.allclose(s, np.sqrt(c / d), rtol=1e-6)
    up2, dn2 = O.apply_smoothing(up, dn, s)
    target = np.sqrt(c * d)
    assert np.allclose(np.linalg.norm(up2.astype(np.float64), axis=1), target, rtol=1e-5)
    assert np.allclose(np.linalg.norm(dn2.astype(np.float64), axis=0), target, rtol=1e-5)


def check_smoothing_max_norm():
    up = np.zeros((3, 8)); dn = np.zeros((5, 3))
    up[0, 2], up[1, 7], up[2, 0] = -8.0, 2.0, 0.5
    dn[4, 0], dn[0, 1], dn[2, 2] = 2.0, -0.5, 0.5
    up[0, 3], dn[1, 0] = 1.0, 0.1   # smaller entries do not change the max
    s = O.smoothing_scales(up, dn, "max")
    assert s.tolist() == [2.0, 2.0, 1.0]


def check_smoothing_zero_channel():
    up = np.ones((3, 4)); dn = np.ones((4, 3))   # equal norms (2) where nothing is zero
    up[1] = 0.0
    dn[:, 2] = 0.0
    assert O.smoothing_scales(up, dn, "l2").tolist() == [1.0, 1.0, 1.0]


def check_smoothing_preserves_gated_ffn(seed: int = 15):
    """y = W_down (gelu(W_gate x) * (W_up x)) is unchanged by smoothing."""
    from scipy.special import erf
    g = np.random.default_rng(seed)
    F, K = 64, 48
    x = g.standard_normal((5, K))
    Wg = g.standard_normal((F, K))
    Wu = g.standard_normal((F, K)) * np.exp(g.standard_normal(F))[:, None]
    Wd = g.standard_normal((K, F)) * np.exp(g.standard_normal(F))[None, :]
    gelu = lambda t: 0.5 * t * (1 + erf(t / np.sqrt(2)))
    ffn = lambda wu, wd: (gelu(x @ Wg.T) * (x @ np.asarray(wu, np.float64).T)) @ np.asarray(wd, np.float64).T
    s = O.smoothing_scales(Wu, Wd, "l2")
    assert np.max(np.abs(s - 1)) > 0.1
    up2, dn2 = O.apply_smoothing(Wu, Wd, s)
    y0, y1 = ffn(Wu.astype(np.float32), Wd.astype(np.float32)), ffn(up2, dn2)
    assert np.linalg.norm(y1 - y0) <= 1e-5 * np.linalg.norm(y0)



# -- runtime LoRA correction ------------------------------------------------------

def check_lora_merged_identity(seed: int = 16):
    """On small integers (exact in bf16 and in the products), the correction
    equals the linear with the merged weight scale B A minus the base."""
    g = np.random.default_rng(seed)
    X = g.integers(-3, 4, (5, 32)).astype(np.float32)
    A = g.integers(-2, 3, (4, 32)).astype(np.float32)
    B = g.integers(-2, 3, (24, 4)).astype(np.float32)
    W = g.integers(-5, 6, (24, 32)).astype(np.float32)
    scale = 0.5
    merged = O.linear_unquantized64(X, W + scale * (B.astype(np.float64) @ A.astype(np.float64)))
    base = O.linear_unquantized64(X, W)
    assert np.array_equal(base + O.lora_delta64(X, A, B, scale), merged)


def check_lora_one_hot():
    X = np.zeros((2, 16), np.float32); X[0, 3] = 2.0; X[1, 7] = -1.0
    A = np.zeros((2, 16), np.float32); A[1, 3] = 0.25; A[0, 7] = 4.0
    B = np.zeros((5, 2), np.float32); B[2, 1] = 3.0; B[4, 0] = -1.0
    d = O.lora_delta64(X, A, B, 2.0)
    want = np.zeros((2, 5)); want[0, 2] = 2.0 * (2.0 * 0.25) * 3.0; want[1, 4] = 2.0 * (-4.0) * -1.0
    assert np.array_equal(d, want)


def check_lora_intermediate_rounds_to_bf16():
    # 1 + 2^-9 is below half a bf16 ulp above 1 (ulp 2^-7): it rounds to 1;
    # 1 + 3 * 2^-8 rounds up to 1 + 2^-6 (ties and nearest, bf16 keeps 8 bits).
    X = np.array([[1.0, 2.0 ** -9], [1.0, 3 * 2.0 ** -8]], np.float32)
    A = np.array([[1.0, 1.0]], np.float32)
    T = O.lora_intermediate(X, A)
    assert T[:, 0].tolist() == [1.0, 1.0 + 2.0 ** -6]


def check_lora_bruteforce(seed: int = 17):
    g = np.random.default_rng(seed)
    X = g.standard_normal((3, 16)).astype(np.float32)
    A = g.standard_normal((2, 16)).astype(np.float32)
    B = g.standard_normal((4, 2)).astype(np.float32)
    T = O.lora_intermediate(X, A).astype(np.float64)
    for m in range(3):
        for j in range(2):
            t = sum(float(X[m, k]) * float(A[j, k]) for k in range(16))
            assert T[m, j] == O.bf16_round(np.array([t], np.float32))[0]
    d = O.lora_delta64(X, A, B, 0.75)
    for m in range(3):
        for n in range(4):
            ref = 0.75 * sum(T[m, j] * float(B[n, j]) for j in range(2))
            assert abs(d[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


ALL_CHECKS = [
    ("r4_printed", check_r4_printed, ()),
    *[(f"regular_structure_G{G}", check_regular_structure, (G,)) for G in REGULAR_GS],
    *[(f"regular_closed_form_G{G}", check_regular_closed_form, (G,)) for G in (4, 16, 64, 256)],
    *[(f"sylvester_G{G}", check_sylvester, (G,)) for G in (2, 16, 128, 1024)],
    *[(f"randomized_orthonormal_G{G}", check_randomized_orthonormal, (G,)) for G in (16, 128)],
    *[(f"block_placement_G{G}", check_rotate_block_placement, (G, 4 * G)) for G in (4, 16, 64, 256)],
    ("randomized_onehot_order", check_randomized_onehot_order, (128, 384)),
    *[(f"invariance_G{G}", check_invariance, (G, O.REGULAR, 2 * G)) for G in REGULAR_GS],
    ("invariance_randomized", check_invariance, (128, O.RANDOMIZED, 1152)),
    *[(f"parseval_G{G}", check_parseval, (G, O.REGULAR, 2 * G)) for G in (16, 256)],
    ("parseval_randomized", check_parseval, (128, O.RANDOMIZED, 256)),
    *[(f"onehot_spreading_G{G}", check_onehot_spreading, (G,)) for G in REGULAR_GS],
    *[(f"constant_row_G{G}", check_constant_row_fixed_point, (G,)) for G in (4, 256)],
    ("quant_invariants", check_quant_invariants, ()),
    ("quant_ties_half_even", check_quant_ties_half_even, ()),
    ("qmax_from_pages", check_qmax_from_pages, ()),
    ("code_values", check_code_values, ()),
    ("group_absmax", check_group_absmax, ()),
    ("int_gemm_bruteforce", check_int_gemm_bruteforce, ()),
    ("int_gemm_extremes", check_int_gemm_extremes, ()),
    ("int_gemm_large_random", check_int_gemm_large_random, ()),
    ("epilogue_scalar", check_epilogue_scalar, ()),
    *[(f"onehot_linear_G{G}", check_onehot_linear_closed_form, (G,)) for G in (4, 16, 256)],
    ("bf16_round", check_bf16_round, ()),
    ("fallback_bruteforce", check_fallback_bruteforce, ()),
    ("routing", check_routing, ()),
    ("qmax4_from_pages", check_qmax4_from_pages, ()),
    ("int4_ties_half_even", check_int4_ties_half_even, ()),
    ("int4_invariants", check_int4_invariants, ()),
    ("nibble_worked_example", check_nibble_worked_example, ()),
    ("nibble_bytes_exhaustive", check_nibble_bytes_exhaustive, ()),
    ("int4_rotation_correlation", check_int4_rotation_correlation, ()),
    ("w4a8_int_gemm_bruteforce", check_w4a8_int_gemm_bruteforce, ()),
    ("smoothing_closed_form", check_smoothing_closed_form, ()),
    ("smoothing_max_norm", check_smoothing_max_norm, ()),
    ("smoothing_zero_channel", check_smoothing_zero_channel, ()),
    ("smoothing_preserves_gated_ffn", check_smoothing_preserves_gated_ffn, ()),
    ("lora_merged_identity", check_lora_merged_identity, ()),
    ("lora_one_hot", check_lora_one_hot, ()),
    ("lora_intermediate_bf16", check_lora_intermediate_rounds_to_bf16, ()),
    ("lora_bruteforce", check_lora_bruteforce, ()),
]


def run_all() -> list[str]:
    """Run every check; return the names of those that fail."""
    failed = []
    for name, fn, args in ALL_CHECKS:
        try:
            fn(*args)
        except Exception:  # noqa: BLE001 - a planted mistake may raise anything
            failed.append(name)
    return failed
