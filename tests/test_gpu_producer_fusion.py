"""Producer fusion of the next layer's pack (convrot_linear_act_rowmax +
convrot_pack_act_rowmax): the up projection's epilogue also emits, per row
and per group of the next layer's G, the largest magnitude of its rotated
output, and the next pack takes the row maximum from those instead of
reducing the row.

* Y equals convrot_linear_act's Y bit for bit (same expression).
* The group maxima equal, bit for bit, the maxima of the GPU's own rotation
  of Y (convrot_rotate, the pack kernel's arithmetic), and the oracle's
  group_absmax of its fp64 rotation of Y within the rotation tolerance
  (1e-5 of the row's largest magnitude).
* The pack from the given maxima equals convrot_pack_act on Y bit for bit
  (codes and scales), and the oracle's pack of Y within the code rules.
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


def _layer(M, N, K, seed, cuda):
    x = random_rows((M, K), seed, dtype="bf16")
    x[:, 7] *= 30.0   # an outlier channel, rounded back to bf16 values
    x = to_bf16_values(x)
    w = random_rows((N, K), seed + 1, sigma=0.02, dtype="bf16")
    b = random_rows((N,), seed + 2, sigma=0.01)
    pa = cr.pack_act(to_dev(x, torch.bfloat16), 64)   # this layer's own rotation (G = 64 divides every K here)
    pw = cr.pack_weight(to_dev(w, torch.bfloat16), 64)
    return pa, pw, to_dev(b, torch.float32)


@pytest.mark.parametrize("M,N,K,G", [(300, 512, 1024, 256), (17, 256, 1024, 16), (513, 768, 2048, 64),
                                     (600, 1280, 3072, 4), (256, 256, 128, 256)])
@pytest.mark.parametrize("act", [cr.GELU_ERF, cr.GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_rowmax_and_prescaled_pack(cuda, M, N, K, G, act, out):
    pa, pw, b = _layer(M, N, K, M + N + K + G, cuda)
    y_ref = cr.linear_act(pa, pw, b, act, out_dtype=out)
    y, pm = cr.linear_act_rowmax(pa, pw, G, b, act, out_dtype=out)
    assert torch.equal(y, y_ref)
    # maxima of the GPU's own rotation of Y: bit-exact
    xr = cr.rotate(y, G)
    own = torch.amax(torch.abs(xr).view(M, N // G, G), dim=2)
    assert torch.equal(pm, own)
    # against the oracle's fp64 rotation of the same Y
    y_np = to_np(y).astype(np.float32)
    ref = O.group_absmax(O.rotate(y_np, G), G)
    row = np.max(ref, axis=1, keepdims=True)
    assert np.all(np.abs(to_np(pm) - ref) <= R.ROT_RTOL * np.where(row > 0, row, 1.0))
    # the pack from the given maxima
    p1 = cr.pack_act(y, G)
    p2 = cr.pack_act_rowmax(y, pm, G)
    assert torch.equal(p2.q, p1.q) and torch.equal(p2.scale, p1.scale)
    q_ref, s_ref, xr_ref = O.pack(y_np, G)
    rep = R.compare_codes(to_np(p2.q), q_ref, O.code_values(xr_ref, s_ref))
    assert rep.ok(), str(rep)
    assert R.scale_rel_diff(to_np(p2.scale), s_ref) <= R.SCALE_RTOL


def test_rowmax_zero_rows_and_strided_buffers(cuda):
    """Rows of zeros give zero maxima and scale 0; strided Y and maxima
    buffers keep their padding."""
    M, N, K, G = 40, 512, 1024, 64
    pa, pw, _ = _layer(M, N, K, 5, cuda)
    pa.q[3].zero_()
    pa.scale[3] = 0.0
    ybuf = torch.full((M, N + 64), 7.0, dtype=torch.bfloat16, device=cuda)
    pbuf = torch.full((M, N // G + 8), -1.0, dtype=torch.float32, device=cuda)
    # no bias: a zero activation row gives a zero output row
    y, pm = cr.linear_act_rowmax(pa, pw, G, None, cr.GELU_ERF, out=ybuf[:, 32:32 + N],
                                 rowmax=pbuf[:, 4:4 + N // G])
    assert torch.all(ybuf[:, :32] == 7.0) and torch.all(ybuf[:, 32 + N:] == 7.0)
    assert torch.all(pbuf[:, :4] == -1.0) and torch.all(pbuf[:, 4 + N // G:] == -1.0)
    assert torch.all(pm[3] == 0)
    p2 = cr.pack_act_rowmax(y, pm, G)
    assert p2.scale[3].item() == 0.0 and torch.all(p2.q[3] == 0)
    p1 = cr.pack_act(y.contiguous(), G)
    assert torch.equal(p2.q, p1.q) and torch.equal(p2.scale, p1.scale)


def test_rowmax_rejects_unsupported_shapes(cuda):
    pa, pw, b = _layer(64, 320, 1024, 9, cuda)
    with pytest.raises(cr.ConvrotError, match="256"):
        cr.linear_act_rowmax(pa, pw, 64, b)                    # N % 256 != 0
    pa16, pw2, b2 = _layer(16, 256, 1024, 10, cuda)
    with pytest.raises(cr.ConvrotError, match="M >"):
        cr.linear_act_rowmax(pa16, pw2, 64, b2)                # small M runs the weight-streaming kernel
    pa3, pw3, b3 = _layer(64, 256, 1024, 11, cuda)
    with pytest.raises(cr.ConvrotError):
        cr.linear_act_rowmax(pa3, pw3, 128, b3)                # not a regular group size
