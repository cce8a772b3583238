"""int4 ConvRot weights on the int8 activation path (W4A8).

What is compared (stable-diffusion.cpp PR "load ConvRot int4 and per-channel
int8 safetensors", sections "Solution" and "The rotation"; the oracle's int4
functions restate them):

* the int4 pack against the oracle's: codes under the same tie rule as the
  int8 codes, scales to 1e-5, and the nibble bytes exactly;
* the in-register and the workspace expansion of nibbles against the
  oracle's decoder, bit-exact over every byte value;
* the W4A8 linear (small-M weight streaming with in-register expansion, and
  the expanded-weight tiled path) against the oracle's exact int32
  accumulator and fp64 epilogue, plain, with an activation, and gated;
* the same call against the int8 linear on the expanded codes: identical
  bits, since accumulators and epilogue are shared.
"""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import rademacher, random_codes, random_codes4, random_rows, to_bf16_values

pytestmark = pytest.mark.gpu


def _w4(q4: np.ndarray, s: np.ndarray, G: int, kind=cr.REGULAR, signs=None) -> cr.PackedW4:
    return cr.PackedW4(to_dev(O.pack_nibbles(q4), torch.uint8), to_dev(s, torch.float32), q4.shape[1], G, kind,
                       signs)


def _operands(M, N, K, seed):
    g = np.random.default_rng(seed)
    qx, q4 = random_codes((M, K), seed), random_codes4((N, K), seed + 1)
    sx = g.uniform(0.5, 1.5, M).astype(np.float32) / np.float32(127.0 * np.sqrt(K))
    sw = g.uniform(0.5, 1.5, N).astype(np.float32) * np.float32(3.0 / 7.0)
    b = (g.standard_normal(N) * 0.5).astype(np.float32)
    return qx, sx, q4, sw, b


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G,K,N", [(4, 64, 5), (16, 1152, 37), (64, 1152, 30), (256, 3072, 19), (1024, 6144, 3),
                                   (256, 12288, 4), (256, 65536, 2)])
def test_pack_weight_w4_regular(cuda, G, K, N, dtype):
    w = random_rows((N, K), seed=G + K + N, dtype="f32")
    g = np.random.default_rng(K + N)
    w.reshape(-1)[g.choice(N * K, size=max(1, N * K // 200), replace=False)] *= 40.0
    if dtype == "bf16":
        w = to_bf16_values(w)
    wd = to_dev(w, torch.bfloat16 if dtype == "bf16" else torch.float32)
    p = cr.pack_weight_w4(wd, G)
    b_ref, s_ref, q_ref, wr = O.pack_weight_int4(w, G)
    q_gpu = O.unpack_nibbles(to_np(p.q))
    rep = R.compare_codes(q_gpu, q_ref, O.code_values(wr, s_ref), qmax=O.QMAX4)
    print(rep)
    assert rep.ok(), rep
    assert np.max(np.abs(q_gpu)) <= 7
    assert R.scale_rel_diff(to_np(p.scale), s_ref) <= R.SCALE_RTOL
    if rep.differ == 0:
        assert np.array_equal(to_np(p.q), b_ref)


@pytest.mark.parametrize("G,K,N", [(128, 1152, 9), (16, 1152, 3), (1024, 6144, 2)])
def test_pack_weight_w4_randomized(cuda, G, K, N):
    w = to_bf16_values(random_rows((N, K), seed=3 * G + K, dtype="f32"))
    signs = rademacher(G + K, K)
    sd = to_dev(signs, torch.int8)
    p = cr.pack_weight_w4(to_dev(w, torch.bfloat16), G, cr.RANDOMIZED, sd)
    _, s_ref, q_ref, wr = O.pack_weight_int4(w, G, O.RANDOMIZED, signs)
    rep = R.compare_codes(O.unpack_nibbles(to_np(p.q)), q_ref, O.code_values(wr, s_ref), qmax=O.QMAX4)
    assert rep.ok(), rep
    assert R.scale_rel_diff(to_np(p.scale), s_ref) <= R.SCALE_RTOL


def test_pack_weight_w4_zero_row_and_strided_output(cuda):
    K, N, G = 512, 6, 64
    w = random_rows((N, K), seed=5)
    w[3] = 0.0
    buf = torch.full((N, K // 2 + 32), 0xAB, dtype=torch.uint8, device=cuda)
    out = cr.PackedW4(buf[:, 16:16 + K // 2], torch.empty(N, dtype=torch.float32, device=cuda), K, G)
    cr.pack_weight_w4(to_dev(w, torch.float32), G, out=out)
    _, s_ref, q_ref, _ = O.pack_weight_int4(w, G)
    assert to_np(out.scale)[3] == 0 and not np.any(to_np(out.q)[3])
    assert torch.all(buf[:, :16] == 0xAB) and torch.all(buf[:, 16 + K // 2:] == 0xAB)


def test_unpack_every_byte(cuda):
    rows, K = 5, 512
    b = (np.arange(rows * K // 2) % 256).astype(np.uint8).reshape(rows, K // 2)
    np.random.default_rng(1).shuffle(b, axis=1)
    w = cr.PackedW4(to_dev(b, torch.uint8), torch.ones(rows, dtype=torch.float32, device=cuda), K, 256)
    assert np.array_equal(to_np(cr.unpack_w4(w)), O.unpack_nibbles(b))


SHAPES = [
    # (M, N, K): small M (weight streaming, incl. the split-K path and K
    # tails inside a 64-feature step), then the expanded-weight tiled path
    (1, 520, 1024), (4, 6912, 1152), (16, 1152, 6912), (16, 300, 1040), (7, 33, 4096),
    (17, 260, 1024), (300, 520, 2064), (513, 1000, 3072),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_linear_w4(cuda, M, N, K):
    qx, sx, q4, sw, b = _operands(M, N, K, M * 31 + N + K)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    w = _w4(q4, sw, 16)
    A = O.int_gemm(qx, q4)
    assert np.array_equal(to_np(cr.linear_w4(a, w, out_dtype=torch.int32)), A)
    bd = to_dev(b, torch.float32)
    y64 = O.epilogue64(A, sx, sw, b)
    y32 = to_np(cr.linear_w4(a, w, bd, out_dtype=torch.float32))
    assert R.rel_fro(y32, y64) <= 1e-5
    ybf = to_np(cr.linear_w4(a, w, bd, out_dtype=torch.bfloat16))
    assert np.array_equal(ybf, O.bf16_round(y32))
    # identical bits to the int8 linear on the expanded codes
    w8 = cr.Packed(cr.unpack_w4(w), w.scale, 16)
    assert np.array_equal(to_np(cr.linear(a, w8, bd, out_dtype=torch.float32)), y32)


@pytest.mark.parametrize("M,N,K", [(4, 6912, 1152), (16, 300, 1040), (300, 520, 2064)])
@pytest.mark.parametrize("act", [cr.GELU_ERF, cr.GELU_TANH])
def test_linear_w4_act_and_gated(cuda, M, N, K, act):
    qx, sx, qg, sg, bg = _operands(M, N, K, 3 * M + N)
    _, _, qu, su, bu = _operands(M, N, K, 5 * M + N + 1)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    wg, wu = _w4(qg, sg, 16), _w4(qu, su, 16)
    bgd, bud = to_dev(bg, torch.float32), to_dev(bu, torch.float32)
    g64 = O.epilogue64(O.int_gemm(qx, qg), sx, sg, bg)
    u64 = O.epilogue64(O.int_gemm(qx, qu), sx, su, bu)
    y = to_np(cr.linear_w4(a, wg, bgd, act, out_dtype=torch.float32))
    assert R.rel_fro(y, R.gelu64(g64, act)) <= 1e-5
    gated = to_np(cr.linear_w4_gated(a, wg, wu, bgd, bud, act, out_dtype=torch.float32))
    assert R.rel_fro(gated, R.gelu64(g64, act) * u64) <= 1e-5
    w8g, w8u = cr.Packed(cr.unpack_w4(wg), wg.scale, 16), cr.Packed(cr.unpack_w4(wu), wu.scale, 16)
    assert np.array_equal(gated, to_np(cr.linear_gated(a, w8g, w8u, bgd, bud, act, out_dtype=torch.float32)))


def test_w4a8_decode_layer_full_size(cuda):
    """The decode FFN at its real shape (M = 16, G = 64: gate/up [6912, 1152],
    down [1152, 6912]) from float weights and activations through the int4
    pack, against the oracle end to end."""
    M, K, N, G = 16, 1152, 6912, 64
    g = np.random.default_rng(77)
    x = to_bf16_values(g.standard_normal((M, K)).astype(np.float32))
    Wg = to_bf16_values((g.standard_normal((N, K)) * 0.03).astype(np.float32))
    Wu = to_bf16_values((g.standard_normal((N, K)) * 0.03).astype(np.float32))
    Wd = to_bf16_values((g.standard_normal((K, N)) * 0.03).astype(np.float32))
    pg, pu, pd = (cr.pack_weight_w4(to_dev(w, torch.bfloat16), G) for w in (Wg, Wu, Wd))
    a = cr.pack_act(to_dev(x, torch.bfloat16), G)
    h = cr.linear_w4_gated(a, pg, pu, act=cr.GELU_TANH, out_dtype=torch.bfloat16)
    y = to_np(cr.linear_w4(cr.pack_act(h, G), pd, out_dtype=torch.float32))
    # oracle, with the GPU's own packed codes where floating point decided them
    qx = to_np(a.q)
    qg, qu, qd = (O.unpack_nibbles(to_np(p.q)) for p in (pg, pu, pd))
    for W, p, q in ((Wg, pg, qg), (Wu, pu, qu), (Wd, pd, qd)):
        _, s_ref, q_ref, wr = O.pack_weight_int4(W, G)
        assert R.compare_codes(q, q_ref, O.code_values(wr, s_ref), qmax=O.QMAX4).ok()
    g64 = O.epilogue64(O.int_gemm(qx, qg), to_np(a.scale), to_np(pg.scale))
    u64 = O.epilogue64(O.int_gemm(qx, qu), to_np(a.scale), to_np(pu.scale))
    h_ref = O.bf16_round((R.gelu64(g64, cr.GELU_TANH) * u64).astype(np.float32))
    assert R.rel_fro(to_np(h), h_ref) <= R.Y_RTOL
    ah = cr.pack_act(h, G)
    y_ref = O.epilogue64(O.int_gemm(to_np(ah.q), qd), to_np(ah.scale), to_np(pd.scale))
    assert R.rel_fro(y, y_ref) <= 1e-5


@pytest.mark.parametrize("M,N,K", [(16, 16400, 1024), (3, 17000, 2080), (1, 16384, 512)])
def test_small_m_two_tile_workgroups(cuda, M, N, K):
    """Small M with at least four 16-feature tiles per CU (256 CUs): the
    weight-streaming kernel computes two tiles per workgroup (int8, int4 and
    bf16 weights; ragged last pair)."""
    qx, sx, q4, sw, b = _operands(M, N, K, N + K)
    q8 = random_codes((N, K), N + K + 2)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    assert np.array_equal(to_np(cr.linear_w4(a, _w4(q4, sw, 16), out_dtype=torch.int32)), O.int_gemm(qx, q4))
    w8 = cr.Packed(to_dev(q8, torch.int8), to_dev(sw, torch.float32), 16)
    assert np.array_equal(to_np(cr.linear(a, w8, out_dtype=torch.int32)), O.int_gemm(qx, q8))
    bd = to_dev(b, torch.float32)
    y = to_np(cr.linear_w4(a, _w4(q4, sw, 16), bd, cr.GELU_ERF, out_dtype=torch.float32))
    assert R.rel_fro(y, R.gelu64(O.epilogue64(O.int_gemm(qx, q4), sx, sw, b), "gelu_erf")) <= 1e-5
    xb = to_bf16_values(random_rows((M, K), 3))
    wb = to_bf16_values(random_rows((N, K), 4) * np.float32(0.05))
    yb = to_np(cr.linear_bf16(to_dev(xb, torch.bfloat16), to_dev(wb, torch.bfloat16), out_dtype=torch.float32))
    assert R.rel_fro(yb, O.linear_unquantized64(xb, wb)) <= 1e-5


@pytest.mark.parametrize("M,N,K", [(16, 3200, 8192), (8, 2000, 4112), (5, 6912, 1152), (16, 1300, 3136),
                                   (2, 17000, 2080)])
def test_small_m_int8_staged_weights(cuda, M, N, K):
    """int8 weights staged through LDS in whole lines (waves streaming five
    or more K steps): with split K (3200 x 8192), K tails inside a two-step
    round (4112, 3136), odd step counts per wave, and two tiles per
    workgroup (17000); plain and gated, against the exact accumulator."""
    qx, sx, _, sw, b = _operands(M, N, K, 7 * N + K)
    qg, qu = random_codes((N, K), N + 5), random_codes((N, K), N + 6)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    wg = cr.Packed(to_dev(qg, torch.int8), to_dev(sw, torch.float32), 16)
    wu = cr.Packed(to_dev(qu, torch.int8), to_dev(sw, torch.float32), 16)
    assert np.array_equal(to_np(cr.linear(a, wg, out_dtype=torch.int32)), O.int_gemm(qx, qg))
    ws = cr.linear_workspace("plain", M, N, K, cuda)   # split K where the shape allows
    assert np.array_equal(to_np(cr.linear(a, wg, out_dtype=torch.int32, workspace=ws)), O.int_gemm(qx, qg))
    g64 = O.epilogue64(O.int_gemm(qx, qg), sx, sw)
    u64 = O.epilogue64(O.int_gemm(qx, qu), sx, sw)
    y = to_np(cr.linear_gated(a, wg, wu, act=cr.GELU_TANH, out_dtype=torch.float32))
    assert R.rel_fro(y, R.gelu64(g64, "gelu_tanh") * u64) <= 1e-5


@pytest.mark.parametrize("M,N,K", [(16, 3200, 8192), (5, 6912, 4096), (12, 9000, 5152), (3, 17000, 2080)])
def test_small_m_int4_staged_weights(cuda, M, N, K):
    """int4 weights staged through LDS in whole lines (waves streaming five
    or more 128-code units, K % 32 == 0): a long K (3200 x 8192; int4 never
    splits K, so the workspace query returns none), a K tail
    inside a unit with ragged N (9000 x 5152), two tiles per workgroup
    (17000); plain and gated, against the exact accumulator."""
    qx, sx, qg, sw, _ = _operands(M, N, K, 11 * N + K)
    qu = random_codes4((N, K), N + 9)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 16)
    wg, wu = _w4(qg, sw, 16), _w4(qu, sw, 16)
    assert np.array_equal(to_np(cr.linear_w4(a, wg, out_dtype=torch.int32)), O.int_gemm(qx, qg))
    assert cr.linear_workspace("w4", M, N, K, cuda) is None
    g64 = O.epilogue64(O.int_gemm(qx, qg), sx, sw)
    u64 = O.epilogue64(O.int_gemm(qx, qu), sx, sw)
    y = to_np(cr.linear_w4_gated(a, wg, wu, act=cr.GELU_TANH, out_dtype=torch.float32))
    assert R.rel_fro(y, R.gelu64(g64, "gelu_tanh") * u64) <= 1e-5



@pytest.mark.parametrize("M,N,K", [(3, 5, 16), (1, 1, 32), (20, 7, 48), (0, 9, 64), (16, 33, 16)])
def test_linear_w4_edges(cuda, M, N, K):
    """Smallest K (one 16-code chunk), a single output, M = 0, and the
    expanded-weight path at tiny sizes."""
    qx, sx, q4, sw, b = _operands(max(M, 1), N, K, 3 * N + K + M)
    qx, sx = qx[:M], sx[:M]
    a = cr.Packed(to_dev(qx.reshape(M, K), torch.int8), to_dev(sx, torch.float32), 16)
    y = cr.linear_w4(a, _w4(q4, sw, 16), out_dtype=torch.int32)
    assert tuple(y.shape) == (M, N)
    if M:
        assert np.array_equal(to_np(y), O.int_gemm(qx, q4))
