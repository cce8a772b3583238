"""Fused epilogues of the quantised linear: an activation applied in the
epilogue (convrot_linear_act) and the gated pair act(gate) * up over one
packed activation (convrot_linear_gated), on the small-M and the tiled
kernels.

References: the oracle's exact int32 accumulator and fp64 epilogue, then the
activation evaluated in fp64 from its definition (scipy's erf, numpy's tanh).
The activation is not part of the method the oracle restates; it is the
layer that follows the linear (a GELU MLP, a gated feed-forward layer), so
it lives with the comparison rules (tests/parity.py, pinned against torch's
GELU in the CPU suite).
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_codes

pytestmark = pytest.mark.gpu


gelu64 = R.gelu64


def operands(M, N, K, seed, with_bias=True):
    g = np.random.default_rng(seed)
    qx, qw = random_codes((M, K), seed), random_codes((N, K), seed + 1)
    # scales that put Y in GELU's curved range (|y| of a few units)
    sx = g.uniform(0.5, 1.5, M).astype(np.float32) / np.float32(127.0 * np.sqrt(K))
    sw = g.uniform(0.5, 1.5, N).astype(np.float32) * np.float32(3.0 / 127.0)
    b = (g.standard_normal(N) * 0.5).astype(np.float32) if with_bias else None
    return qx, sx, qw, sw, b


def packed(q, s, G):
    return cr.Packed(to_dev(q, torch.int8), to_dev(s, torch.float32), G)


SHAPES = [
    # (M, N, K): small-M kernel, then the tiled kernel with ragged tails
    (1, 520, 1024), (4, 6912, 1152), (16, 300, 1040),
    (17, 260, 1024), (300, 520, 2064), (513, 1000, 3072),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("act", [cr.GELU_ERF, cr.GELU_TANH])
def test_linear_act(cuda, M, N, K, act):
    G = 16
    qx, sx, qw, sw, b = operands(M, N, K, M + 7 * N)
    y64 = O.epilogue64(O.int_gemm(qx, qw), sx, sw, b)
    ref = gelu64(y64, act)
    a, w = packed(qx, sx, G), packed(qw, sw, G)
    bd = to_dev(b, torch.float32)
    y32 = to_np(cr.linear_act(a, w, bd, act, out_dtype=torch.float32))
    err = R.rel_fro(y32, ref)
    assert err <= 1e-5, err
    ybf = to_np(cr.linear_act(a, w, bd, act, out_dtype=torch.bfloat16))
    assert R.rel_fro(ybf, O.bf16_round(ref.astype(np.float32))) <= R.Y_RTOL
    # bf16 outputs are the RNE rounding of the kernel's own fp32 outputs
    assert np.array_equal(ybf, O.bf16_round(y32))
    # with a workspace small M may split K: the same result bits
    ws = cr.linear_workspace("plain", M, N, K, cuda)
    if ws is not None:
        assert np.array_equal(to_np(cr.linear_act(a, w, bd, act, out_dtype=torch.float32, workspace=ws)), y32)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("act", [cr.GELU_TANH, cr.GELU_ERF])
def test_linear_gated(cuda, M, N, K, act):
    G = 16
    qx, sx, qg, sg, bg = operands(M, N, K, 3 * M + N)
    _, _, qu, su, bu = operands(M, N, K, 5 * M + N + 1)
    g64 = O.epilogue64(O.int_gemm(qx, qg), sx, sg, bg)
    u64 = O.epilogue64(O.int_gemm(qx, qu), sx, su, bu)
    ref = gelu64(g64, act) * u64
    a, wg, wu = packed(qx, sx, G), packed(qg, sg, G), packed(qu, su, G)
    bgd, bud = to_dev(bg, torch.float32), to_dev(bu, torch.float32)
    y32 = to_np(cr.linear_gated(a, wg, wu, bgd, bud, act, out_dtype=torch.float32))
    assert R.rel_fro(y32, ref) <= 1e-5
    ybf = to_np(cr.linear_gated(a, wg, wu, bgd, bud, act, out_dtype=torch.bfloat16))
    assert R.rel_fro(ybf, O.bf16_round(ref.astype(np.float32))) <= R.Y_RTOL
    assert np.array_equal(ybf, O.bf16_round(y32))
    ws = cr.linear_workspace("gated", M, N, K, cuda)
    if ws is not None:
        y_split = cr.linear_gated(a, wg, wu, bgd, bud, act, out_dtype=torch.float32, workspace=ws)
        assert np.array_equal(to_np(y_split), y32)


def test_gated_without_bias_and_strided_output(cuda):
    M, N, K, G = 40, 200, 512, 64
    qx, sx, qg, sg, _ = operands(M, N, K, 11, with_bias=False)
    _, _, qu, su, _ = operands(M, N, K, 12, with_bias=False)
    ref = gelu64(O.epilogue64(O.int_gemm(qx, qg), sx, sg), cr.GELU_TANH) * O.epilogue64(O.int_gemm(qx, qu), sx, su)
    buf = torch.full((M, N + 24), -3.0, dtype=torch.float32, device=cuda)
    cr.linear_gated(packed(qx, sx, G), packed(qg, sg, G), packed(qu, su, G), out=buf[:, 8:8 + N])
    assert R.rel_fro(to_np(buf[:, 8:8 + N]), ref) <= 1e-5
    assert torch.all(buf[:, :8] == -3.0) and torch.all(buf[:, 8 + N:] == -3.0)


def test_gated_equals_two_linears(cuda):
    """One gated launch equals the two plain linears combined afterwards."""
    M, N, K, G = 96, 640, 2048, 256
    qx, sx, qg, sg, bg = operands(M, N, K, 21)
    _, _, qu, su, bu = operands(M, N, K, 22)
    a, wg, wu = packed(qx, sx, G), packed(qg, sg, G), packed(qu, su, G)
    bgd, bud = to_dev(bg, torch.float32), to_dev(bu, torch.float32)
    fused = cr.linear_gated(a, wg, wu, bgd, bud, cr.GELU_TANH, out_dtype=torch.float32)
    g = cr.linear(a, wg, bgd, out_dtype=torch.float32)
    u = cr.linear(a, wu, bud, out_dtype=torch.float32)
    two = torch.nn.functional.gelu(g, approximate="tanh") * u
    assert torch.allclose(fused, two, rtol=1e-5, atol=1e-6)
