"""The TILE16 weight layout read by the small-M (M <= 16) kernels.

tile_weight / tile_weight_w4 rearrange packed weight rows into tiles of 16
rows in which each 64-byte unit of a row's bytes (64 int8 codes, or 128 int4
codes) sits with the same unit of the other 15 rows: 16 x 64 bytes = 1 KiB of
consecutive memory per unit of a tile.  Only addresses change, so:

* the copy is checked byte for byte against that permutation written with
  numpy (int8 and int4, padded source rows) and against the stated byte
  address on sampled bytes; the scales are copied unchanged;
* every small-M entry point on a tiled weight (plain with and without the K
  split, with an activation, gated, int4 plain and gated, the no-allocation
  variant) returns the same bits as on the ROWS weight, and its int32
  accumulator equals the oracle's exact integer product;
* the decode FFN at its full size, in the benchmark's launch configuration
  (tiled weights, split-K workspaces), matches the ROWS weights bit for bit
  and the oracle's gated output within the output gate.
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
import workloads as W
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_codes, random_codes4

pytestmark = pytest.mark.gpu


def tile16(b: np.ndarray) -> np.ndarray:
    """Rows of bytes [N, R] (N % 16 == 0, R % 64 == 0) in the TILE16 order."""
    N, R = b.shape
    return b.reshape(N // 16, 16, R // 64, 64).transpose(0, 2, 1, 3).reshape(N, R)


def tiled_offset(r: int, byte: int, row_bytes: int) -> int:
    """Address of byte ``byte`` of row ``r`` in a TILE16 weight."""
    return (r // 16) * 16 * row_bytes + (byte // 64) * 1024 + (r % 16) * 64 + byte % 64


def _scales(n, seed):
    return np.random.default_rng(seed).uniform(0.5, 1.5, n).astype(np.float32) / np.float32(127.0)


@pytest.mark.parametrize("N,K", [(16, 64), (48, 1152), (1152, 6912), (6912, 1152), (64, 8192)])
def test_tile_weight_is_the_stated_permutation(cuda, N, K):
    q = random_codes((N, K), N + K)
    s = _scales(N, K)
    buf = torch.zeros((N, K + 96), dtype=torch.int8, device=cuda)     # padded source rows (ld = K + 96)
    buf[:, 32:32 + K] = to_dev(q, torch.int8)
    w = cr.Packed(buf[:, 32:32 + K], to_dev(s, torch.float32), 16)
    t = cr.tile_weight(w)
    assert t.layout == cr.TILE16 and tuple(t.q.shape) == (N, K) and t.q.is_contiguous()
    got = to_np(t.q)
    assert np.array_equal(got, tile16(q))
    flat = got.reshape(-1)
    g = np.random.default_rng(N * K)
    for r, b in zip(g.integers(0, N, 256), g.integers(0, K, 256)):
        assert flat[tiled_offset(int(r), int(b), K)] == q[r, b]
    assert np.array_equal(to_np(t.scale), s)


@pytest.mark.parametrize("N,K", [(16, 128), (6912, 1152), (1152, 6912)])
def test_tile_weight_w4_is_the_stated_permutation(cuda, N, K):
    q4 = random_codes4((N, K), N + K)
    nib = O.pack_nibbles(q4)
    s = _scales(N, K + 1)
    w = cr.PackedW4(to_dev(nib, torch.uint8), to_dev(s, torch.float32), K, 16)
    t = cr.tile_weight_w4(w)
    assert t.layout == cr.TILE16
    assert np.array_equal(to_np(t.q), tile16(nib))
    assert np.array_equal(to_np(t.scale), s)


def test_tile_weight_rejects_a_tiled_input(cuda):
    w = cr.Packed(to_dev(random_codes((16, 64), 1), torch.int8), torch.ones(16, device=cuda), 16)
    t = cr.tile_weight(w)
    with pytest.raises(ValueError, match="ROWS"):
        cr.tile_weight(t)
    a = cr.Packed(to_dev(random_codes((17, 64), 2), torch.int8), torch.ones(17, device=cuda), 16)
    with pytest.raises(RuntimeError, match="M <= 16"):
        cr.linear(a, t)


SHAPES = [(16, 3200, 8192), (5, 6912, 1152), (1, 16384, 512), (16, 1152, 6912), (3, 17008, 2048),
          (12, 9008, 5248)]


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_tiled_int8_weights_give_the_same_bits(cuda, M, N, K):
    seed = 13 * N + K + M
    qx, qg, qu = random_codes((M, K), seed), random_codes((N, K), seed + 1), random_codes((N, K), seed + 2)
    sx, sg, su = _scales(M, seed), _scales(N, seed + 1), _scales(N, seed + 2)
    b = to_dev((np.random.default_rng(seed).standard_normal(N) * 0.5).astype(np.float32), torch.float32)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    wg = cr.Packed(to_dev(qg, torch.int8), to_dev(sg, torch.float32), 16)
    wu = cr.Packed(to_dev(qu, torch.int8), to_dev(su, torch.float32), 16)
    tg, tu = cr.tile_weight(wg), cr.tile_weight(wu)
    acc = cr.linear(a, tg, out_dtype=torch.int32)
    assert np.array_equal(to_np(acc), O.int_gemm(qx, qg))
    ws = cr.linear_workspace("plain", M, N, K, cuda)
    for dt in (torch.int32, torch.bfloat16):
        assert _same(cr.linear(a, tg, b, out_dtype=dt, workspace=ws), cr.linear(a, wg, b, out_dtype=dt, workspace=ws))
    assert _same(cr.linear(a, tg, b), cr.linear(a, wg, b))
    assert _same(cr.linear_act(a, tg, b, cr.GELU_ERF, workspace=ws), cr.linear_act(a, wg, b, cr.GELU_ERF, workspace=ws))
    wsg = cr.linear_workspace("gated", M, N, K, cuda)
    for w_s in (None, wsg):
        y_t = cr.linear_gated(a, tg, tu, b, None, cr.GELU_TANH, out_dtype=torch.float32, workspace=w_s)
        y_r = cr.linear_gated(a, wg, wu, b, None, cr.GELU_TANH, out_dtype=torch.float32, workspace=w_s)
        assert _same(y_t, y_r)
    ref = R.gelu64(O.epilogue64(O.int_gemm(qx, qg), sx, sg, to_np(b)), "gelu_tanh") * O.epilogue64(
        O.int_gemm(qx, qu), sx, su)
    assert R.rel_fro(to_np(y_t), ref) <= 1e-5


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_tiled_int4_weights_give_the_same_bits(cuda, M, N, K):
    seed = 17 * N + K + M
    qx, qg, qu = random_codes((M, K), seed), random_codes4((N, K), seed + 1), random_codes4((N, K), seed + 2)
    sx, sg, su = _scales(M, seed), _scales(N, seed + 1), _scales(N, seed + 2)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    wg = cr.PackedW4(to_dev(O.pack_nibbles(qg), torch.uint8), to_dev(sg, torch.float32), K, 16)
    wu = cr.PackedW4(to_dev(O.pack_nibbles(qu), torch.uint8), to_dev(su, torch.float32), K, 16)
    tg, tu = cr.tile_weight_w4(wg), cr.tile_weight_w4(wu)
    assert np.array_equal(to_np(cr.linear_w4(a, tg, out_dtype=torch.int32)), O.int_gemm(qx, qg))
    assert _same(cr.linear_w4(a, tg), cr.linear_w4(a, wg))
    assert _same(cr.linear_w4(a, tg, act=cr.GELU_ERF), cr.linear_w4(a, wg, act=cr.GELU_ERF))
    ws = cr.linear_workspace("w4_gated", M, N, K, cuda)
    y_t = cr.linear_w4_gated(a, tg, tu, act=cr.GELU_TANH, out_dtype=torch.float32, workspace=ws)
    assert _same(y_t, cr.linear_w4_gated(a, wg, wu, act=cr.GELU_TANH, out_dtype=torch.float32, workspace=ws))
    ref = R.gelu64(O.epilogue64(O.int_gemm(qx, qg), sx, sg), "gelu_tanh") * O.epilogue64(O.int_gemm(qx, qu), sx, su)
    assert R.rel_fro(to_np(y_t), ref) <= 1e-5


def test_tiled_weight_on_the_no_allocation_entry_point(cuda):
    M, N, K = 16, 1152, 6912
    qx, qw = random_codes((M, K), 5), random_codes((N, K), 6)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(_scales(M, 5), torch.float32), 64)
    w = cr.Packed(to_dev(qw, torch.int8), to_dev(_scales(N, 6), torch.float32), 64)
    t = cr.tile_weight(w)
    for dt in (torch.int32, torch.bfloat16):
        y_t = cr.linear_noalloc(a, t, torch.empty((M, N), dtype=dt, device=cuda))
        assert _same(y_t, cr.linear_noalloc(a, w, torch.empty((M, N), dtype=dt, device=cuda)))
    assert np.array_equal(to_np(cr.linear_noalloc(a, t, torch.empty((M, N), dtype=torch.int32, device=cuda))),
                          O.int_gemm(qx, qw))


XSHAPES = [(1, 1152, 6912, 64, torch.bfloat16), (3, 17008, 2048, 256, torch.float32),
           (5, 6912, 1152, 64, torch.bfloat16), (8, 640, 64, 64, torch.bfloat16),
           (12, 9008, 5248, 16, torch.bfloat16), (16, 3200, 8192, 256, torch.float32),
           (16, 1152, 6912, 64, torch.bfloat16), (5, 1000, 4096, 64, torch.bfloat16)]


@pytest.mark.parametrize("M,N,K,G,dt", XSHAPES)
def test_tiled_activation_gives_the_same_bits(cuda, M, N, K, G, dt):
    """pack_act(layout=TILE16) writes the TILE16 permutation of the ROWS
    codes (one 16-row tile), and every int8-weight small-M call reading it
    returns the bits it returns for the ROWS activation."""
    seed = 19 * N + K + M
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal((M, K)).astype(np.float32)).to(cuda).to(dt)
    a = cr.pack_act(x, G)
    at = cr.pack_act(x, G, layout=cr.TILE16)
    assert at.layout == cr.TILE16 and tuple(at.q.shape) == (M, K)
    assert torch.equal(at.scale, a.scale)
    full = to_np(at.q.as_strided((16, K), (K, 1)))
    pad = np.zeros((16 - M, K), dtype=np.int8)
    exp = tile16(np.vstack([to_np(a.q), pad]))
    mask = tile16(np.vstack([np.ones((M, K), dtype=np.int8), pad])).astype(bool)
    assert np.array_equal(full[mask], exp[mask])

    qg, qu = random_codes((N, K), seed + 1), random_codes((N, K), seed + 2)
    wg = cr.Packed(to_dev(qg, torch.int8), to_dev(_scales(N, seed + 1), torch.float32), G)
    wu = cr.Packed(to_dev(qu, torch.int8), to_dev(_scales(N, seed + 2), torch.float32), G)
    b = to_dev((g.standard_normal(N) * 0.5).astype(np.float32), torch.float32)
    ws = cr.linear_workspace("plain", M, N, K, cuda)
    wsg = cr.linear_workspace("gated", M, N, K, cuda)
    assert np.array_equal(to_np(cr.linear(at, wg, out_dtype=torch.int32)), O.int_gemm(to_np(a.q), qg))
    tiled = N % 16 == 0
    for w, u in ((wg, wu), (cr.tile_weight(wg), cr.tile_weight(wu))) if tiled else ((wg, wu),):
        for w_s in (None, ws):
            for odt in (torch.int32, torch.float32, torch.bfloat16):
                assert _same(cr.linear(at, w, b, out_dtype=odt, workspace=w_s),
                             cr.linear(a, w, b, out_dtype=odt, workspace=w_s))
            assert _same(cr.linear_act(at, w, b, cr.GELU_ERF, workspace=w_s),
                         cr.linear_act(a, w, b, cr.GELU_ERF, workspace=w_s))
        for w_s in (None, wsg):
            assert _same(cr.linear_gated(at, w, u, b, None, cr.GELU_TANH, out_dtype=torch.float32, workspace=w_s),
                         cr.linear_gated(a, w, u, b, None, cr.GELU_TANH, out_dtype=torch.float32, workspace=w_s))
        for odt in (torch.int32, torch.bfloat16):
            assert _same(cr.linear_noalloc(at, w, torch.empty((M, N), dtype=odt, device=cuda), b),
                         cr.linear_noalloc(a, w, torch.empty((M, N), dtype=odt, device=cuda), b))


def test_tiled_activation_is_refused_where_it_is_not_read(cuda):
    x = torch.randn(17, 256, device=cuda)
    with pytest.raises(ValueError, match="M <= 16"):
        cr.pack_act(x, 64, layout=cr.TILE16)
    with pytest.raises(ValueError, match="K % 64"):
        cr.pack_act(x[:4, :96], 16, layout=cr.TILE16)
    at = cr.pack_act(x[:4], 64, layout=cr.TILE16)
    w4 = cr.pack_weight_w4(torch.randn(64, 256, device=cuda), 64)
    with pytest.raises(RuntimeError, match="ROWS"):
        cr.linear_w4(at, w4)


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 16])
def test_decode_ffn_tiled_full(cuda, M):
    """The decode FFN (X [M, 1152], gate and up [6912, 1152], down
    [1152, 6912], G = 64) as the benchmark launches it by default: tiled
    weights, the gated launch and the down linear each with its split-K
    workspace.  Identical bits to the ROWS weights; the gated output within
    the output gate of the oracle's."""
    G = 64
    wl = W.config5(M=M, G=G, kind="regular")
    gate, up, down = wl.linears
    pa = cr.pack_act(to_dev(wl.X, torch.bfloat16), G)
    pg, pu, pd = (cr.pack_weight(to_dev(l.W, torch.bfloat16 if l.wdtype == "bf16" else torch.float32), G)
                  for l in (gate, up, down))
    tg, tu, td = cr.tile_weight(pg), cr.tile_weight(pu), cr.tile_weight(pd)
    bg, bu, bd = (to_dev(l.b, torch.float32) for l in (gate, up, down))
    wsg = cr.linear_workspace("gated", M, 6912, 1152, cuda)
    h_t = cr.linear_gated(pa, tg, tu, bg, bu, cr.GELU_TANH, workspace=wsg)
    h_r = cr.linear_gated(pa, pg, pu, bg, bu, cr.GELU_TANH, workspace=wsg)
    assert _same(h_t, h_r)
    qx, sx = to_np(pa.q), to_np(pa.scale)
    ref = O.bf16_round((R.gelu64(O.epilogue64(O.int_gemm(qx, to_np(pg.q)), sx, to_np(pg.scale), gate.b), "gelu_tanh")
                        * O.epilogue64(O.int_gemm(qx, to_np(pu.q)), sx, to_np(pu.scale), up.b)).astype(np.float32))
    err = R.rel_fro(to_np(h_t), ref)
    print(f"decode M={M}: gated rel Frobenius {err:.3e}", flush=True)
    assert err <= R.Y_RTOL
    ph = cr.pack_act(h_t, G)
    wsd = cr.linear_workspace("plain", M, 1152, 6912, cuda)
    assert _same(cr.linear(ph, td, bd, workspace=wsd), cr.linear(ph, pd, bd, workspace=wsd))
    assert np.array_equal(to_np(cr.linear(ph, td, out_dtype=torch.int32, workspace=wsd)),
                          O.int_gemm(to_np(ph.q), to_np(pd.q)))


@pytest.mark.parametrize("bits", [8, 4])
def test_layer_tiled_for_decode(cuda, bits):
    """ConvRotLinear.tile_for_decode: same bits as the ROWS layer for M <= 16
    (a merged pair too), an error for more rows."""
    from w8a8_int8_linear_amd.layer import ConvRotLinear
    g = torch.Generator(device="cpu").manual_seed(bits)
    w1 = (torch.randn(96, 1152, generator=g) * 0.02).to(cuda)
    w2 = (torch.randn(64, 1152, generator=g) * 0.02).to(cuda)
    b1 = (torch.randn(96, generator=g) * 0.01).to(cuda)
    x = torch.randn(7, 1152, generator=g).to(cuda, torch.bfloat16)
    rows = [ConvRotLinear.from_dense(w, b, 64, weight_bits=bits) for w, b in ((w1, b1), (w2, None))]
    tiled = [ConvRotLinear.from_dense(w, b, 64, weight_bits=bits) for w, b in ((w1, b1), (w2, None))]
    for l in tiled:
        l.tile_for_decode()
        assert l.packed.layout == cr.TILE16
    for r, t in zip(rows, tiled):
        assert _same(t(x), r(x))
    mr, mt = ConvRotLinear.merge(rows), ConvRotLinear.merge(tiled)
    assert _same(mt(x), mr(x))
    with pytest.raises(RuntimeError, match="M <= 16"):
        tiled[0](torch.randn(17, 1152, generator=g).to(cuda, torch.bfloat16))
