"""The routed unquantised path (K % G != 0) and the layer-level routing."""

import logging

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(300, 520, 2688), (37, 100, 64), (513, 1024, 1040), (5, 7, 16), (1, 300, 2688),
                                   # M <= 16: the weight-streaming kernel (one or several load rounds, K tails)
                                   (16, 1152, 6912), (4, 6912, 1152), (16, 33, 1040), (2, 24, 16384)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_linear_bf16_parity(cuda, M, N, K, out):
    x = random_rows((M, K), M + K, dtype="bf16")
    w = random_rows((N, K), N + K, sigma=0.02, dtype="bf16")
    b = random_rows((N,), N, sigma=0.01)
    ref64 = O.linear_unquantized64(x, w, b)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    y = to_np(cr.linear_bf16(to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16), to_dev(b, torch.float32), od))
    ref = O.bf16_round(ref64.astype(np.float32)) if out == "bf16" else ref64
    err = R.rel_fro(y, ref)
    assert err <= R.Y_RTOL, err
    if out == "f32":
        assert err <= 1e-5, err
    ws = cr.linear_workspace("bf16", M, N, K, cuda)
    if ws is not None:   # small M, K split: fp32 partials added in K order
        ys = to_np(cr.linear_bf16(to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16), to_dev(b, torch.float32), od,
                                  workspace=ws))
        assert R.rel_fro(ys, ref) <= (1e-5 if out == "f32" else R.Y_RTOL)


def test_routing_and_summary(cuda, caplog):
    """A width-2688 layer stays in bf16 (2688 % 256 != 0) and is logged; a
    width-3072 layer packs; both reproduce X W^T + b."""
    routing = cr.RoutingLog()
    caplog.set_level(logging.WARNING, logger="w8a8_int8_linear_amd")
    w1 = to_dev(random_rows((512, 2688), 1, sigma=0.02, dtype="bf16"), torch.bfloat16)
    w2 = to_dev(random_rows((512, 3072), 2, sigma=0.02, dtype="bf16"), torch.bfloat16)
    b = torch.zeros(512, device=cuda)
    l1 = cr.ConvRotLinear.from_dense(w1, b, 256, name="adaln", routing=routing)
    l2 = cr.ConvRotLinear.from_dense(w2, b, 256, name="qkv", routing=routing)
    assert not l1.quantized and l2.quantized
    assert [(r.layer, r.K, r.path) for r in routing.routes] == [("adaln", 2688, "bf16"), ("qkv", 3072, "int8")]
    assert routing.by_path("bf16")[0].reason == "K = 2688 is not a multiple of G = 256"
    assert "adaln" in caplog.text and "qkv" not in caplog.text
    assert "adaln    2688  bf16" in routing.report()
    x1 = to_dev(random_rows((2, 3, 2688), 3, dtype="bf16"), torch.bfloat16)
    y1 = l1(x1)
    assert y1.shape == (2, 3, 512)
    ref1 = O.linear_unquantized64(to_np(x1).reshape(6, 2688), to_np(w1))
    assert R.rel_fro(to_np(y1).reshape(6, 512), ref1) <= R.Y_RTOL
    x2 = to_dev(random_rows((2, 3, 3072), 4, dtype="bf16"), torch.bfloat16)
    y2 = l2(x2)
    ref2 = O.linear_unquantized64(to_np(x2).reshape(6, 3072), to_np(w2))
    assert R.rel_fro(to_np(y2).reshape(6, 512), ref2) <= 0.05   # quantisation error vs the dense layer
    with pytest.raises(ValueError):
        l1(l2.pack_input(x2))


def test_packed_activation_reuse(cuda):
    """One packed activation feeds two linears; each equals its own call."""
    x = to_dev(random_rows((64, 1024), 5, dtype="bf16"), torch.bfloat16)
    la = cr.ConvRotLinear.from_dense(to_dev(random_rows((300, 1024), 6, sigma=0.02, dtype="bf16"), torch.bfloat16))
    lb = cr.ConvRotLinear.from_dense(to_dev(random_rows((100, 1024), 7, sigma=0.02, dtype="bf16"), torch.bfloat16))
    pa = la.pack_input(x)
    assert torch.equal(la(pa), la(x)) and torch.equal(lb(pa), lb(x))


@pytest.mark.parametrize("bits", [8, 4])
def test_merged_layers_one_launch(cuda, bits):
    """Layers on one input merged into one launch over their stacked packed
    weights: each output is a column view equal bit for bit to the layer's
    own output; packed activations reuse works on the merged layer too."""
    K, G = 1024, 256
    x = to_dev(random_rows((300, K), 31, dtype="bf16"), torch.bfloat16)
    layers = []
    for i, n in enumerate((384, 128, 200)):
        w = to_dev(random_rows((n, K), 40 + i, sigma=0.02, dtype="bf16"), torch.bfloat16)
        b = torch.randn(n, device=cuda) * 0.01 if i != 1 else None
        layers.append(cr.ConvRotLinear.from_dense(w, b, G, name=f"l{i}", weight_bits=bits))
    merged = cr.ConvRotLinear.merge(layers)
    assert merged.N == 712 and merged.splits == [384, 128, 200]
    for m in (300, 7):
        ys = merged.split(merged(x[:m]))
        for l, y in zip(layers, ys):
            assert torch.equal(y, l(x[:m])), (l.name, m)
    pa = merged.pack_input(x)
    assert torch.equal(merged(pa), merged(x))
    twice = cr.ConvRotLinear.merge([merged, layers[0]])
    assert twice.splits == [384, 128, 200, 384]
    assert torch.equal(twice.split(twice(x))[3], layers[0](x))


def test_merge_rejects_mismatched_layers(cuda):
    K = 512
    w = to_dev(random_rows((64, K), 50, sigma=0.02, dtype="bf16"), torch.bfloat16)
    a = cr.ConvRotLinear.from_dense(w, group=256, name="a")
    with pytest.raises(ValueError, match="group"):
        cr.ConvRotLinear.merge([a, cr.ConvRotLinear.from_dense(w, group=64, name="b")])
    with pytest.raises(ValueError, match="weight width"):
        cr.ConvRotLinear.merge([a, cr.ConvRotLinear.from_dense(w, group=256, name="c", weight_bits=4)])
    routed = cr.ConvRotLinear.from_dense(w[:, :500], group=256, name="r")
    with pytest.raises(ValueError, match="routed"):
        cr.ConvRotLinear.merge([a, routed])
    signs = torch.where(torch.arange(K, device=cuda) % 3 == 0, -1, 1).to(torch.int8)
    rz = cr.ConvRotLinear.from_dense(w, group=256, kind=cr.RANDOMIZED, signs=signs, name="z")
    with pytest.raises(ValueError):
        cr.ConvRotLinear.merge([a, rz])
    lo = cr.ConvRotLinear.from_dense(w, group=256, name="lo")
    lo.add_lora(torch.zeros(16, K, device=cuda), torch.zeros(64, 16, device=cuda), 1.0)
    with pytest.raises(ValueError, match="adapters"):
        cr.ConvRotLinear.merge([a, lo])
    with pytest.raises(ValueError):
        cr.ConvRotLinear.merge([])
