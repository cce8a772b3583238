"""The Python binding's own checks (CPU only).  The library takes M and N
from the packed operands and only the row pitch from a caller's output, so
the binding must reject an output that is not exactly [M, N] with unit
column stride before it calls anything; packed descriptors must hold int8
codes with unit stride along K and one fp32 scale per row.  Every case
here raises ValueError before any library call or launch."""

import pytest
import torch

import w8a8_int8_linear_amd as cr


def _packed(rows, K, q_dtype=torch.int8):
    return cr.Packed(torch.zeros((rows, K), dtype=q_dtype), torch.ones(rows, dtype=torch.float32), 256)


@pytest.mark.parametrize("shape", [(31, 64), (32, 63), (64, 64), (32 * 64,)])
def test_linear_rejects_a_wrong_shaped_output(shape):
    a, w = _packed(32, 256), _packed(64, 256)
    with pytest.raises(ValueError, match="shape"):
        cr.linear(a, w, out=torch.empty(shape, dtype=torch.bfloat16))


@pytest.mark.parametrize("fn", ["linear_act", "linear_w4"])
def test_fused_and_int4_linears_reject_a_wrong_shaped_output(fn):
    a = _packed(32, 256)
    if fn == "linear_act":
        w = _packed(64, 256)
        call = lambda out: cr.linear_act(a, w, out=out)  # noqa: E731
    else:
        w = cr.PackedW4(torch.zeros((64, 128), dtype=torch.uint8), torch.ones(64), 256, 256)
        call = lambda out: cr.linear_w4(a, w, out=out)  # noqa: E731
    with pytest.raises(ValueError, match="shape"):
        call(torch.empty((16, 64), dtype=torch.bfloat16))


def test_gated_rejects_a_wrong_shaped_output():
    a, g, u = _packed(8, 256), _packed(64, 256), _packed(64, 256)
    with pytest.raises(ValueError, match="shape"):
        cr.linear_gated(a, g, u, out=torch.empty((8, 32), dtype=torch.bfloat16))


def test_bf16_linear_rejects_a_wrong_shaped_output():
    x = torch.zeros((10, 64), dtype=torch.bfloat16)
    w = torch.zeros((20, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        cr.linear_bf16(x, w, out=torch.empty((9, 20), dtype=torch.bfloat16))


def test_output_needs_unit_column_stride_and_a_known_dtype():
    a, w = _packed(32, 256), _packed(64, 256)
    strided = torch.empty((32, 128), dtype=torch.bfloat16)[:, ::2]
    with pytest.raises(ValueError, match="stride"):
        cr.linear(a, w, out=strided)
    with pytest.raises(ValueError, match="dtype"):
        cr.linear(a, w, out=torch.empty((32, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="dtype"):
        cr.linear_act(a, w, out=torch.empty((32, 64), dtype=torch.int32))


def test_bias_must_match_n():
    a, w = _packed(32, 256), _packed(64, 256)
    with pytest.raises(ValueError, match="bias"):
        cr.linear(a, w, torch.zeros(63), out=torch.empty((32, 64), dtype=torch.bfloat16))


def test_descriptor_checks_codes_and_scales():
    with pytest.raises(ValueError, match="int8"):
        _packed(4, 256, torch.int32).descriptor()
    q = torch.zeros((4, 512), dtype=torch.int8)[:, ::2]
    with pytest.raises(ValueError, match="unit stride"):
        cr.Packed(q, torch.ones(4), 256).descriptor()
    with pytest.raises(ValueError, match="scales"):
        cr.Packed(torch.zeros((4, 256), dtype=torch.int8), torch.ones(3), 256).descriptor()
    # well-formed, but host memory: the library only takes device tensors
    with pytest.raises(ValueError, match="device"):
        _packed(4, 256).descriptor()
