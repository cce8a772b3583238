"""Data-free smoothing of an FFN's intermediate channels (gemma.cpp issue
"Add experimental W8A8 MatMul with optional QuaRot-style rotation", the
maintainer's review comment; the oracle's smoothing functions restate it).

* The scales s against the oracle's fp64 computation (within one fp32 ulp),
  for both norms, bf16 and fp32 weights, a zero channel and strided inputs.
* The scaled weights against the oracle's fp64 quotient / product with the
  GPU's own s: bit-exact.
* The study the comment asks for: quantisation error of a gated FFN with
  imbalanced intermediate channels (moderate and strong imbalance), through the whole GPU path (pack, gated
  linear, pack, linear), against the unquantised fp64 layer, for G = 64 and
  256, int8 and int4 weights, with and without smoothing.  Smoothing must
  not lose accuracy on this input; the table is printed.
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_rows, smoothing_study_ffn, to_bf16_values

pytestmark = pytest.mark.gpu


def _ulp_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.abs(b)))


@pytest.mark.parametrize("norm", ["l2", "max"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("F,K,Ko", [(96, 256, 64), (1000, 1152, 300), (8192, 3072, 3072)])
def test_smoothing_matches_oracle(cuda, norm, dtype, F, K, Ko):
    g = np.random.default_rng(F + K)
    up = random_rows((F, K), F, dtype="f32") * np.exp(g.standard_normal(F)).astype(np.float32)[:, None]
    dn = random_rows((Ko, F), K, dtype="f32") * np.exp(g.standard_normal(F)).astype(np.float32)[None, :]
    up[3] = 0.0
    dn[:, 5] = 0.0
    if dtype == "bf16":
        up, dn = to_bf16_values(up), to_bf16_values(dn)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s, up2, dn2 = cr.smooth_ffn(to_dev(up, tdt), to_dev(dn, tdt), norm)
    s_np = to_np(s)
    s_ref = O.smoothing_scales(up, dn, norm)
    assert s_np[3] == 1.0 and s_np[5] == 1.0
    assert _ulp_rel(s_np, s_ref) <= 2.0 ** -23
    up_ref, dn_ref = O.apply_smoothing(up, dn, s_np)
    assert np.array_equal(to_np(up2), up_ref)
    assert np.array_equal(to_np(dn2), dn_ref)


def test_smoothing_strided_inputs_and_scales_only(cuda):
    F, K, Ko = 64, 128, 80
    up = to_bf16_values(random_rows((F, K + 32), 1))
    dn = to_bf16_values(random_rows((Ko, F + 16), 2))
    upd, dnd = to_dev(up, torch.bfloat16)[:, :K], to_dev(dn, torch.bfloat16)[:, :F]
    s = to_np(cr.smooth_ffn(upd, dnd, "l2", scaled=False))
    assert _ulp_rel(s, O.smoothing_scales(up[:, :K], dn[:, :F], "l2")) <= 2.0 ** -23


def _ffn_error(X, Wg, Wu, Wd, G, bits, norm, cuda):
    bf = torch.bfloat16
    wg, wu, wd = to_dev(Wg, bf), to_dev(Wu, bf), to_dev(Wd, bf)
    if norm is not None:
        _, wu, wd = cr.smooth_ffn(wu, wd, norm)
    pack = cr.pack_weight if bits == 8 else cr.pack_weight_w4
    pg, pu, pd = pack(wg, G), pack(wu, G), pack(wd, G)
    a = cr.pack_act(to_dev(X, bf), G)
    if bits == 8:
        h = cr.linear_gated(a, pg, pu, act=cr.GELU_TANH, out_dtype=bf)
        y = cr.linear(cr.pack_act(h, G), pd, out_dtype=torch.float32)
    else:
        h = cr.linear_w4_gated(a, pg, pu, act=cr.GELU_TANH, out_dtype=bf)
        y = cr.linear_w4(cr.pack_act(h, G), pd, out_dtype=torch.float32)
    return to_np(y)


@pytest.mark.parametrize("sigma_c", [0.5, 1.5])
def test_smoothing_study(cuda, sigma_c):
    X, Wg, Wu, Wd = smoothing_study_ffn(sigma_c=sigma_c)
    x64 = X.astype(np.float64)
    h64 = R.gelu64(x64 @ Wg.astype(np.float64).T, "gelu_tanh") * (x64 @ Wu.astype(np.float64).T)
    y64 = h64 @ Wd.astype(np.float64).T
    rows = []
    errs = {}
    for bits in (8, 4):
        for G in (64, 256):
            for norm in (None, "max", "l2"):
                e = R.rel_fro(_ffn_error(X, Wg, Wu, Wd, G, bits, norm, cuda), y64)
                errs[(bits, G, norm)] = e
                rows.append(f"sigma_c={sigma_c} W{bits}A8 G={G:4d} smoothing={str(norm):5s} rel Frobenius error "
                            f"{e:.4e}")
    print("\n" + "\n".join(rows))
    for bits in (8, 4):
        for G in (64, 256):
            assert errs[(bits, G, "l2")] < errs[(bits, G, None)]
