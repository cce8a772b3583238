"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""

import numpy as np
import pytest

import oracle.convrot_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("name,fn,args", P.ALL_CHECKS, ids=[c[0] for c in P.ALL_CHECKS])
def test_pin(name, fn, args):
    fn(*args)


def test_row_split_is_bit_exact():
    """Rows are independent: packing row chunks equals packing the whole
    (sglang summary page, large-M row split is bit-exact)."""
    g = np.random.default_rng(11)
    X = g.standard_normal((37, 512)).astype(np.float32)
    q, s, xr = O.pack(X, 256)
    parts = [O.pack(X[a:b], 256) for a, b in ((0, 8), (8, 30), (30, 37))]
    assert np.array_equal(q, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(s, np.concatenate([p[1] for p in parts]))


def test_forgotten_rotation_is_noise():
    """Rotated weights used with unrotated activations give output with no
    useful correlation to the true layer ("feat: load ConvRot int4 ...",
    section "The rotation": ignoring the rotation produces noise)."""
    g = np.random.default_rng(12)
    K, N, M = 1024, 256, 64
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    truth = X.astype(np.float64) @ W.astype(np.float64).T
    qw, sw, _ = O.pack(W, 256)
    good = O.linear(X, qw, sw, None, 256)["y64"]
    qx_raw, sx_raw = O.quantize_rows(X)
    bad = O.epilogue64(O.int_gemm(qx_raw, qw), sx_raw, sw)
    corr = lambda a, b: float(np.corrcoef(a.ravel(), b.ravel())[0, 1])
    assert corr(good, truth) > 0.999
    assert abs(corr(bad, truth)) < 0.1


def test_rotation_reduces_outlier_error():
    """With isolated outliers the rotated W8A8 output is closer to X W^T than
    the unrotated one ("INT8 Convrot Safetensors": the rotation spreads large
    values across each group).  Informational property, not a parity gate."""
    from workloads import config1
    wl = config1()
    W = wl.linears[0].W
    truth = O.linear_unquantized64(wl.X, W)
    qw, sw, _ = O.pack(W, 256)
    rot = O.linear(wl.X, qw, sw, None, 256)["y64"]
    qx0, sx0 = O.quantize_rows(wl.X)
    qw0, sw0 = O.quantize_rows(W)
    plain = O.epilogue64(O.int_gemm(qx0, qw0), sx0, sw0)
    e_rot = np.linalg.norm(rot - truth) / np.linalg.norm(truth)
    e_plain = np.linalg.norm(plain - truth) / np.linalg.norm(truth)
    assert e_rot < 0.5 * e_plain, (e_rot, e_plain)


def test_input_domain_errors():
    with pytest.raises(ValueError):
        O.regular_rotation(8)
    with pytest.raises(ValueError):
        O.rotate64(np.zeros((1, 100)), 64)
    with pytest.raises(ValueError):
        O.rotate64(np.full((1, 16), np.nan), 16)
    with pytest.raises(ValueError):
        O.rotate64(np.zeros((1, 128)), 128, O.RANDOMIZED, None)
    with pytest.raises(TypeError):
        O.quantize_rows(np.zeros((1, 4)))
