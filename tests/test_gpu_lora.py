"""Runtime LoRA correction ("INT8 Convrot Safetensors", LoRA paragraph; the
oracle's lora functions restate it): dY = scale (X A^T) B^T from the
unrotated activation, added in place to the base output.

* The rank-r intermediate (left in the workspace) against the oracle's
  fp64 product rounded to bf16: within one bf16 ulp.
* The added correction against scale T B^T of the GPU's own T in fp64:
  within 1e-5 relative Frobenius (fp32 accumulation over r), ragged M and
  N, ranks 16 to 256.
* A whole layer: the int8 ConvRot linear of the packed input plus the
  adapter, against the oracle's quantised linear plus its correction.
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_rows, to_bf16_values

pytestmark = pytest.mark.gpu


def _adapter(M, K, N, r, seed):
    g = np.random.default_rng(seed)
    x = to_bf16_values(random_rows((M, K), seed))
    a = to_bf16_values((g.standard_normal((r, K)) * (1.0 / np.sqrt(K))).astype(np.float32))
    b = to_bf16_values((g.standard_normal((N, r)) * 0.05).astype(np.float32))
    return x, a, b


@pytest.mark.parametrize("M,K,N,r", [(1, 1024, 520, 16), (16, 1152, 6912, 32), (17, 256, 100, 16),
                                     (300, 3072, 1000, 64), (513, 2048, 777, 128), (70, 1040, 64, 256),
                                     (33, 512, 300, 48), (20, 512, 130, 64), (9, 1024, 200, 128),
                                     (128, 2048, 96, 32)])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_lora_add(cuda, M, K, N, r, ydt):
    x, a, b = _adapter(M, K, N, r, M + K + N + r)
    scale = 0.75
    xd, ad, bd = (to_dev(t, torch.bfloat16) for t in (x, a, b))
    tdt = torch.float32 if ydt == "f32" else torch.bfloat16
    y0 = random_rows((M, N), 5)
    if ydt == "bf16":
        y0 = to_bf16_values(y0)
    y = to_dev(y0, tdt)
    ws = torch.empty((cr.lora_workspace_bytes(M, K, r) + 1) // 2, dtype=torch.bfloat16, device=cuda)
    cr.lora_add(xd, ad, bd, scale, y, workspace=ws)
    # the call leaves its bf16 intermediate T [M, r] at the workspace's start
    T = to_np(ws[:M * r].view(M, r))
    T_ref = O.lora_intermediate(x, a)
    assert np.all(np.abs(T - T_ref) <= np.abs(T_ref) * 2.0 ** -7 + 1e-30)
    got = to_np(y).astype(np.float64)
    delta = float(np.float32(scale)) * (T.astype(np.float64) @ b.astype(np.float64).T)
    if ydt == "f32":
        assert R.rel_fro(got - y0, delta) <= 1e-5
    else:
        want = O.bf16_round((y0.astype(np.float64) + delta).astype(np.float32))
        assert R.rel_fro(got, want) <= 2e-3
        assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-3)) <= 2.0 ** -7


def test_lora_add_strided_output_and_untouched_padding(cuda):
    M, K, N, r = 40, 512, 200, 16
    x, a, b = _adapter(M, K, N, r, 9)
    buf = torch.full((M, N + 24), -3.0, dtype=torch.float32, device=cuda)
    y = buf[:, 8:8 + N]
    y.zero_()
    ws = torch.empty((cr.lora_workspace_bytes(M, K, r) + 1) // 2, dtype=torch.bfloat16, device=cuda)
    cr.lora_add(*(to_dev(t, torch.bfloat16) for t in (x, a, b)), 2.0, y, workspace=ws)
    T = to_np(ws[:M * r].view(M, r)).astype(np.float64)
    got = to_np(y).astype(np.float64)
    # the added correction is 2 T B^T of the call's own T, summed in fp32 over r
    assert R.rel_fro(got, 2.0 * (T @ b.astype(np.float64).T)) <= 1e-5
    # against the oracle: T is within one bf16 ulp (2^-7 relative) plus the
    # worst-case fp32 summation error K 2^-24 sum |x a| of its K products, so
    # |dY| <= 2 (dT |B|^T) elementwise, plus the fp32 sum over r
    T_ref = O.lora_intermediate(x, a).astype(np.float64)
    dT = np.abs(T_ref) * 2.0 ** -7 + K * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(a.astype(np.float64)).T)
    assert np.all(np.abs(T - T_ref) <= dT)
    ref = O.lora_delta64(x, a, b, 2.0)
    bound = np.linalg.norm(2.0 * (dT @ np.abs(b.astype(np.float64)).T)) / np.linalg.norm(ref) + 1e-5
    assert R.rel_fro(got, ref) <= bound
    assert torch.all(buf[:, :8] == -3.0) and torch.all(buf[:, 8 + N:] == -3.0)


def test_convrot_layer_with_adapter(cuda):
    """Base int8 ConvRot linear from the packed (rotated) input plus the
    adapter from the unrotated input."""
    M, K, N, r, G = 64, 3072, 3072, 32, 256
    x, a, b = _adapter(M, K, N, r, 21)
    W = to_bf16_values((np.random.default_rng(22).standard_normal((N, K)) * 0.02).astype(np.float32))
    xd = to_dev(x, torch.bfloat16)
    pa, pw = cr.pack_act(xd, G), cr.pack_weight(to_dev(W, torch.bfloat16), G)
    y = cr.linear(pa, pw, out_dtype=torch.float32)
    cr.lora_add(xd, to_dev(a, torch.bfloat16), to_dev(b, torch.bfloat16), 0.5, y)
    ref = O.linear(x, *O.pack(W, G)[:2], None, G)["y64"] + O.lora_delta64(x, a, b, 0.5)
    assert R.rel_fro(to_np(y), ref) <= R.Y_RTOL


def test_layer_int4_weights_with_adapter(cuda):
    """ConvRotLinear with int4 weights and an attached adapter, on a 3-D
    input: the W4A8 linear of the packed input plus the adapter's
    correction from the unrotated input."""
    B_, S, K, N, r, G = 2, 24, 1024, 640, 16, 256
    g = np.random.default_rng(41)
    x = to_bf16_values(g.standard_normal((B_ * S, K)).astype(np.float32))
    W = to_bf16_values((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = (g.standard_normal(N) * 0.01).astype(np.float32)
    _, a, b = _adapter(1, K, N, r, 42)
    layer = cr.ConvRotLinear.from_dense(to_dev(W, torch.bfloat16), to_dev(bias, torch.float32), G, weight_bits=4)
    layer.add_lora(to_dev(a, torch.bfloat16), to_dev(b, torch.bfloat16), 0.5)
    assert layer.weight_bits == 4 and layer.quantized
    y = layer(to_dev(x, torch.bfloat16).reshape(B_, S, K), out_dtype=torch.float32)
    assert tuple(y.shape) == (B_, S, N)
    nib, s_w, q4, _ = O.pack_weight_int4(W, G)
    qx, sx, _ = O.pack(x, G)
    ref = O.epilogue64(O.int_gemm(qx, O.unpack_nibbles(nib)), sx, s_w, bias) + O.lora_delta64(x, a, b, 0.5)
    assert R.rel_fro(to_np(y).reshape(B_ * S, N), ref) <= R.Y_RTOL
    with pytest.raises(ValueError):
        layer(layer.pack_input(to_dev(x, torch.bfloat16)))
