"""The path under HIP graph capture: a captured step replays to the same bits
as the same launches made eagerly.

Steps captured with torch.cuda.graph: a decode step of a gated
feed-forward layer (pack the activation, gate and up in one gated launch,
pack the product, down projection split over K in a caller-owned
workspace), the same step with int4 weights (also
at a width where the weights are staged through LDS), a DiT-sized step
(one pack shared by two linears, 256-row tiles with ragged edges), and a
linear followed by a LoRA correction.  Each graph is replayed three
times; before each replay the captured input buffer is refilled eagerly,
the same launches run eagerly into separate outputs, and the replay's
outputs must equal them bit for bit (the kernels are deterministic, so any
difference is a capture or replay fault).  Eager work and synchronisation
run between the replays.
"""

import numpy as np
import pytest
import torch

import w8a8_int8_linear_amd as cr
from workloads import random_rows

pytestmark = pytest.mark.gpu


def _weights(shapes, G, seed, dev, bits=8):
    g = np.random.default_rng(seed)
    out = []
    pack = cr.pack_weight if bits == 8 else cr.pack_weight_w4
    for n, k in shapes:
        w = torch.from_numpy((g.standard_normal((n, k)) * 0.05).astype(np.float32)).to(torch.bfloat16).to(dev)
        b = torch.from_numpy((g.standard_normal(n) * 0.1).astype(np.float32)).to(dev)
        out.append((pack(w, G), b))
    return out


def _x(M, K, seed, dev):
    return torch.from_numpy(random_rows((M, K), seed).astype(np.float32)).to(torch.bfloat16).to(dev)


def _decode_step(x, ws, bufs, G):
    (wg, bg), (wu, bu), (wd, bd) = ws
    pa, h, pa2, y, wsp = bufs
    cr.pack_act(x, G, out=pa)
    cr.linear_gated(pa, wg, wu, bg, bu, cr.GELU_TANH, out=h)
    cr.pack_act(h, G, out=pa2)
    cr.linear(pa2, wd, bd, out=y, workspace=wsp)   # down projection: K split in the caller's workspace


def _decode_step_w4(x, ws, bufs, G):
    (wg, bg), (wu, bu), (wd, bd) = ws
    pa, h, pa2, y, wsp = bufs
    cr.pack_act(x, G, out=pa)
    cr.linear_w4_gated(pa, wg, wu, bg, bu, cr.GELU_TANH, out=h)
    cr.pack_act(h, G, out=pa2)
    cr.linear_w4(pa2, wd, bd, out=y, workspace=wsp)


def _decode_bufs(M, K, F, G, dev, kind="plain"):
    def packed(rows, k):
        return cr.Packed(torch.empty((rows, k), dtype=torch.int8, device=dev),
                         torch.empty(rows, dtype=torch.float32, device=dev), G)
    wsp = cr.linear_workspace(kind, M, K, F, dev)   # None where the down projection does not split K
    if kind == "plain" and M == 16:
        assert wsp is not None, "the int8 down projection splits K at 16 rows"
    return (packed(M, K), torch.empty((M, F), dtype=torch.bfloat16, device=dev), packed(M, F),
            torch.empty((M, K), dtype=torch.bfloat16, device=dev), wsp)


def _dit_step(x, ws, bufs, G):
    (w1, b1), (w2, b2) = ws
    pa, y1, y2 = bufs
    cr.pack_act(x, G, out=pa)
    cr.linear(pa, w1, b1, out=y1)
    cr.linear(pa, w2, b2, out=y2)


def _dit_bufs(M, K, N1, N2, G, dev):
    return (cr.Packed(torch.empty((M, K), dtype=torch.int8, device=dev),
                      torch.empty(M, dtype=torch.float32, device=dev), G),
            torch.empty((M, N1), dtype=torch.bfloat16, device=dev),
            torch.empty((M, N2), dtype=torch.bfloat16, device=dev))


def _outputs(bufs):
    """Every output buffer of a step (workspaces are scratch, not outputs)."""
    outs = [b for b in bufs if b is not None and (isinstance(b, cr.Packed) or b.dtype != torch.uint8)]
    return [b.q if isinstance(b, cr.Packed) else b for b in outs] + \
           [b.scale for b in outs if isinstance(b, cr.Packed)]


def _replay_matches_eager(step, make_bufs, ws, M, K, G, seed, dev):
    x = _x(M, K, seed, dev)
    cap = make_bufs()
    ref = make_bufs()
    step(x, ws, cap, G)             # warm-up (first-call set-up happens outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, ws, cap, G)
    for r in range(3):
        x.copy_(_x(M, K, seed + 1 + r, dev))
        step(x, ws, ref, G)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(cap), _outputs(ref)):
            assert torch.equal(a, b), f"replay {r} differs from the eager launches"


@pytest.mark.parametrize("M", [1, 16])
def test_decode_step_graph(cuda, M):
    K, F, G = 1152, 6912, 64
    ws = _weights([(F, K), (F, K), (K, F)], G, 5, cuda)
    _replay_matches_eager(_decode_step, lambda: _decode_bufs(M, K, F, G, cuda), ws, M, K, G, 100 + M, cuda)


def test_dit_step_graph(cuda):
    M, K, N1, N2, G = 600, 1024, 1000, 520, 256
    ws = _weights([(N1, K), (N2, K)], G, 7, cuda)
    _replay_matches_eager(_dit_step, lambda: _dit_bufs(M, K, N1, N2, G, cuda), ws, M, K, G, 200, cuda)


@pytest.mark.parametrize("M,K,F", [(16, 1152, 6912), (4, 4096, 6912)])
def test_decode_step_w4_graph(cuda, M, K, F):
    G = 64
    ws = _weights([(F, K), (F, K), (K, F)], G, 9, cuda, bits=4)
    _replay_matches_eager(_decode_step_w4, lambda: _decode_bufs(M, K, F, G, cuda, "w4"), ws, M, K, G, 300 + M,
                          cuda)


def test_lora_step_graph(cuda):
    M, K, N, r, G = 300, 1024, 700, 32, 256
    ws = _weights([(N, K)], G, 11, cuda)
    g = np.random.default_rng(12)
    a = torch.from_numpy((g.standard_normal((r, K)) / 32).astype(np.float32)).to(torch.bfloat16).to(cuda)
    bu = torch.from_numpy((g.standard_normal((N, r)) * 0.05).astype(np.float32)).to(torch.bfloat16).to(cuda)

    def step(x, ws_, bufs, G_):
        (w, b), = ws_
        pa, y, t = bufs
        cr.pack_act(x, G_, out=pa)
        cr.linear(pa, w, b, out=y)
        cr.lora_add(x, a, bu, 0.5, y, workspace=t)

    def bufs():
        return (cr.Packed(torch.empty((M, K), dtype=torch.int8, device=cuda),
                          torch.empty(M, dtype=torch.float32, device=cuda), G),
                torch.empty((M, N), dtype=torch.bfloat16, device=cuda),
                torch.empty(cr.lora_workspace_bytes(M, K, r), dtype=torch.uint8, device=cuda))
    _replay_matches_eager(step, bufs, ws, M, K, G, 400, cuda)
