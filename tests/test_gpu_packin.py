"""Linears that pack their own activation rows (convrot_linear_packin,
convrot_linear_gated_packin): the rotation, row maximum and quantisation of
the pack ("INT8 Convrot Safetensors", "Runtime activation quantization")
done inside the small-M launch.

What is compared:

* against packing first (pack_act, then linear / linear_act / linear_gated
  on the same weight): identical bits, int32, fp32 and bf16, for every
  regular G in {4, 16, 64, 256, 1024} and the randomized kind (G 16, 128,
  1024), M from 1 to 4, ragged N, K tails, the largest K, strided X and Y,
  TILE16 weights, zero rows and outlier columns;
* the fp32 output against the oracle's fp64 epilogue of the exact integer
  product of the GPU's own codes (within 1e-5), so the epilogue is pinned
  as well as the codes;
* the decode FFN at full size (M = 1 and 4) against the oracle's gated
  output, and its captured graph against eager launches.
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
import workloads as W
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_rows, rademacher, to_bf16_values

pytestmark = pytest.mark.gpu


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _x(M, K, seed, ncols=3):
    x = random_rows((M, K), seed)
    if K > ncols:
        x[:, np.random.default_rng(seed).choice(K, size=ncols, replace=False)] *= np.float32(40.0)
    return to_bf16_values(x)


def _weight(N, K, G, kind, signs, seed, cuda):
    w = to_bf16_values(random_rows((N, K), seed, sigma=0.02))
    return cr.pack_weight(to_dev(w, torch.bfloat16), G, kind, signs)


ROTATIONS = [(4, cr.REGULAR), (16, cr.REGULAR), (64, cr.REGULAR), (256, cr.REGULAR), (1024, cr.REGULAR),
             (16, cr.RANDOMIZED), (128, cr.RANDOMIZED), (1024, cr.RANDOMIZED)]
SHAPES = [(1152, 6912), (6912, 1152), (100, 1040), (520, 16384), (48, 2048), (2000, 4096)]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 4])
def test_packin_equals_pack_then_linear(cuda, M, N, K):
    b = to_dev((np.random.default_rng(N).standard_normal(N) * 0.1).astype(np.float32), torch.float32)
    xn = _x(M, K, 7 * M + K)
    x = to_dev(xn, torch.bfloat16)
    for G, kind in ROTATIONS:
        if K % G:
            continue
        signs = to_dev(rademacher(3, K), torch.int8) if kind == cr.RANDOMIZED else None
        pw = _weight(N, K, G, kind, signs, N + K + G, cuda)
        pa = cr.pack_act(x, G, kind, signs)
        print(f"[packin] M={M} N={N} K={K} G={G} {kind}", flush=True)
        for dt in (torch.int32, torch.float32, torch.bfloat16):
            assert _same(cr.linear_packin(x, pw, None if dt == torch.int32 else b, out_dtype=dt),
                         cr.linear(pa, pw, None if dt == torch.int32 else b, out_dtype=dt)), (G, kind, dt)
        for act in (cr.GELU_ERF, cr.GELU_TANH):
            assert _same(cr.linear_packin(x, pw, b, act=act), cr.linear_act(pa, pw, b, act)), (G, kind, act)
        y = to_np(cr.linear_packin(x, pw, b, out_dtype=torch.float32))
        ref = O.epilogue64(O.int_gemm(to_np(pa.q), to_np(pw.q)), to_np(pa.scale), to_np(pw.scale), to_np(b))
        assert R.rel_fro(y, ref) <= 1e-5
        if N % 16 == 0 and K % 64 == 0:
            assert _same(cr.linear_packin(x, cr.tile_weight(pw), b), cr.linear(pa, pw, b))


@pytest.mark.parametrize("N,K", [(6912, 1152), (100, 1040), (256, 4096)])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_gated_packin_equals_pack_then_gated(cuda, M, N, K):
    rng = np.random.default_rng(N + K)
    bg = to_dev((rng.standard_normal(N) * 0.1).astype(np.float32), torch.float32)
    bu = to_dev((rng.standard_normal(N) * 0.1).astype(np.float32), torch.float32)
    x = to_dev(_x(M, K, 11 * M + K), torch.bfloat16)
    for G, kind in ROTATIONS:
        if K % G:
            continue
        signs = to_dev(rademacher(4, K), torch.int8) if kind == cr.RANDOMIZED else None
        pg = _weight(N, K, G, kind, signs, 2 * N + K, cuda)
        pu = _weight(N, K, G, kind, signs, 3 * N + K, cuda)
        pa = cr.pack_act(x, G, kind, signs)
        print(f"[gated packin] M={M} N={N} K={K} G={G} {kind}", flush=True)
        for act in (cr.GELU_TANH, cr.GELU_ERF):
            for dt in (torch.float32, torch.bfloat16):
                assert _same(cr.linear_gated_packin(x, pg, pu, bg, bu, act, out_dtype=dt),
                             cr.linear_gated(pa, pg, pu, bg, bu, act, out_dtype=dt)), (G, kind, act, dt)
        if N % 16 == 0 and K % 64 == 0:
            tg, tu = cr.tile_weight(pg), cr.tile_weight(pu)
            assert _same(cr.linear_gated_packin(x, tg, tu, bg, bu), cr.linear_gated(pa, pg, pu, bg, bu))


def test_packin_edges(cuda):
    """Zero rows, a row of one value, M = 0, strided X and Y."""
    K, N, G = 2048, 96, 64
    pw = _weight(N, K, G, cr.REGULAR, None, 5, cuda)
    xn = _x(4, K, 9)
    xn[1] = 0.0
    xn[2] = 0.75
    buf = torch.zeros((4, K + 64), dtype=torch.bfloat16, device=cuda)
    buf[:, 32:32 + K] = to_dev(xn, torch.bfloat16)
    xs = buf[:, 32:32 + K]                                   # row pitch K + 64, 64-byte offset
    pa = cr.pack_act(xs, G)
    assert float(pa.scale[1]) == 0.0
    out = torch.full((4, N + 8), 3.0, dtype=torch.float32, device=cuda)
    y = cr.linear_packin(xs, pw, out=out[:, :N], out_dtype=torch.float32)
    assert _same(y, cr.linear(pa, pw, out_dtype=torch.float32))
    assert torch.all(out[:, N:] == 3.0)
    assert tuple(cr.linear_packin(xs[:0], pw).shape) == (0, N)
    with pytest.raises(RuntimeError, match="0 to 4 rows"):
        cr.linear_packin(to_dev(_x(5, K, 1), torch.bfloat16), pw)


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 4])
def test_decode_ffn_packin_full(cuda, M):
    """The decode FFN (X [M, 1152], gate and up [6912, 1152], down
    [1152, 6912], G = 64, TILE16 weights) in two packing launches, as the
    benchmark runs it at M <= 4: identical bits to pack + linear, and the
    gated output within the output gate of the oracle's."""
    G = 64
    wl = W.config5(M=M, G=G, kind="regular")
    gate, up, down = wl.linears
    x = to_dev(wl.X, torch.bfloat16)
    pg, pu, pd = (cr.pack_weight(to_dev(l.W, torch.bfloat16), G) for l in (gate, up, down))
    tg, tu, td = cr.tile_weight(pg), cr.tile_weight(pu), cr.tile_weight(pd)
    bg, bu, bd = (to_dev(l.b, torch.float32) for l in (gate, up, down))
    h = cr.linear_gated_packin(x, tg, tu, bg, bu, cr.GELU_TANH)
    pa = cr.pack_act(x, G)
    assert _same(h, cr.linear_gated(pa, pg, pu, bg, bu, cr.GELU_TANH))
    qx_ref, sx_ref, _ = O.pack(wl.X, G)
    qg_ref, sg_ref, _ = O.pack(gate.W, G)
    qu_ref, su_ref, _ = O.pack(up.W, G)
    ref = O.bf16_round((R.gelu64(O.epilogue64(O.int_gemm(qx_ref, qg_ref), sx_ref, sg_ref, gate.b), "gelu_tanh")
                        * O.epilogue64(O.int_gemm(qx_ref, qu_ref), sx_ref, su_ref, up.b)).astype(np.float32))
    err = R.rel_fro(to_np(h), ref)
    print(f"decode packin M={M}: gated rel Frobenius {err:.3e}", flush=True)
    assert err <= R.Y_RTOL
    y = cr.linear_packin(h, td, bd)
    assert _same(y, cr.linear(cr.pack_act(h, G), pd, bd))


def test_packin_decode_step_graph(cuda):
    """Both packing launches of a decode step captured in a graph: three
    replays, each after refilling the input and running the same launches
    eagerly, equal the eager outputs bit for bit."""
    M, K, F, G = 2, 1152, 6912, 64
    pg, pu = (_weight(F, K, G, cr.REGULAR, None, s, cuda) for s in (1, 2))
    pd = _weight(K, F, G, cr.REGULAR, None, 3, cuda)
    x = torch.empty((M, K), dtype=torch.bfloat16, device=cuda)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=cuda)
    y = torch.empty((M, K), dtype=torch.bfloat16, device=cuda)

    def step():
        cr.linear_gated_packin(x, pg, pu, out=h)
        cr.linear_packin(h, pd, out=y)

    x.copy_(to_dev(_x(M, K, 1), torch.bfloat16))
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        x.copy_(to_dev(_x(M, K, 10 + r), torch.bfloat16))
        step()
        torch.cuda.synchronize()
        eager_h, eager_y = h.clone(), y.clone()
        h.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same(h, eager_h) and _same(y, eager_y), f"replay {r}"
