"""Parity of the quantised linear (tiled MFMA GEMM and small-M kernel) with
the CPU oracle: the int32 accumulator bit-exact, Y within tolerance."""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import config1, random_codes, random_rows

pytestmark = pytest.mark.gpu


def _packed_from_codes(q, s, G, cuda):
    return cr.Packed(to_dev(q, torch.int8), to_dev(s, torch.float32), G)


GEMM_SHAPES = [
    # (M, N, K, G): several 256x256 tiles with ragged M/N tails, K tails
    (300, 520, 1024, 256), (256, 256, 128, 64), (513, 260, 3072, 256), (17, 33, 64, 64),
    (700, 1000, 1040, 16), (64, 1024, 1024, 256), (1000, 300, 12288, 256), (257, 4, 256, 256),
    (40, 8, 1152, 64),
    # small M: the weight-streaming kernel
    (1, 6912, 1152, 64), (4, 1152, 6912, 64), (16, 520, 1024, 256), (3, 17, 80, 16), (16, 16, 64, 4),
    (2, 40, 40960, 256), (16, 100, 16400, 16),
]


@pytest.mark.parametrize("M,N,K,G", GEMM_SHAPES)
def test_accumulator_bit_exact(cuda, M, N, K, G):
    qx = random_codes((M, K), seed=M + 3 * K)
    qw = random_codes((N, K), seed=N + 5 * K)
    sx = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    a, w = _packed_from_codes(qx, sx, G, cuda), _packed_from_codes(qw, sw, G, cuda)
    A_gpu = to_np(cr.linear(a, w, out_dtype=torch.int32))
    A_ref = O.int_gemm(qx, qw)
    assert np.array_equal(A_gpu.astype(np.int64), A_ref)
    # small M with a caller workspace: K split across workgroups, exact int32 partials
    ws = cr.linear_workspace("plain", M, N, K, cuda)
    if ws is not None:
        A_split = to_np(cr.linear(a, w, out_dtype=torch.int32, workspace=ws))
        assert np.array_equal(A_split.astype(np.int64), A_ref)


def test_accumulator_extremes(cuda):
    K = 12288
    qx = np.full((20, K), 127, np.int8)
    qx[1::2] = -127
    qw = np.full((40, K), -127, np.int8)
    qw[::3] = 127
    sx, sw = np.ones(20, np.float32), np.ones(40, np.float32)
    A = to_np(cr.linear(_packed_from_codes(qx, sx, 256, cuda), _packed_from_codes(qw, sw, 256, cuda),
                        out_dtype=torch.int32))
    assert np.array_equal(A.astype(np.int64), O.int_gemm(qx, qw))
    assert np.max(np.abs(A)) == K * 127 * 127


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (16, 520, 1024), (1, 64, 256)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_epilogue_from_oracle_codes(cuda, M, N, K, with_bias):
    G = 256
    g = np.random.default_rng(M + N)
    qx, qw = random_codes((M, K), 1), random_codes((N, K), 2)
    sx = g.uniform(1e-3, 0.1, M).astype(np.float32)
    sw = g.uniform(1e-5, 1e-3, N).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float32) if with_bias else None
    y64 = O.epilogue64(O.int_gemm(qx, qw), sx, sw, b)
    a, w = _packed_from_codes(qx, sx, G, cuda), _packed_from_codes(qw, sw, G, cuda)
    bd = to_dev(b, torch.float32) if with_bias else None
    y32 = to_np(cr.linear(a, w, bd, out_dtype=torch.float32))
    assert R.rel_fro(y32, y64.astype(np.float32)) <= 1e-6
    ybf = to_np(cr.linear(a, w, bd, out_dtype=torch.bfloat16))
    ref_bf = O.bf16_round(y64.astype(np.float32))
    assert R.rel_fro(ybf, ref_bf) <= 1e-3
    # bf16 outputs are the RNE rounding of the kernel's own fp32 outputs
    assert np.array_equal(ybf, O.bf16_round(y32))


def test_persistent_walk_rounds(cuda):
    """More tiles than workgroups: each workgroup of the persistent walk runs
    several tiles, and int8 tiles of alternate rounds take K last slice
    first.  fp32 and bf16 outputs against the oracle's epilogue of the exact
    integer product, as for one round."""
    M, N, K, G = 2048, 18432, 1024, 256
    g = np.random.default_rng(11)
    qx, qw = random_codes((M, K), 5), random_codes((N, K), 6)
    sx = g.uniform(1e-3, 0.1, M).astype(np.float32)
    sw = g.uniform(1e-5, 1e-3, N).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    y64 = O.epilogue64(O.int_gemm(qx, qw), sx, sw, b)
    a, w = _packed_from_codes(qx, sx, G, cuda), _packed_from_codes(qw, sw, G, cuda)
    bd = to_dev(b, torch.float32)
    y32 = to_np(cr.linear(a, w, bd, out_dtype=torch.float32))
    assert R.rel_fro(y32, y64.astype(np.float32)) <= 1e-6
    # every element, against its row's RMS: a tile that skipped or repeated a
    # slice would be off by a sizeable fraction of it
    worst = np.max(np.abs(y32 - y64) / np.sqrt(np.mean(y64 ** 2, axis=1, keepdims=True)))
    assert float(worst) <= 1e-5, float(worst)
    ybf = to_np(cr.linear(a, w, bd, out_dtype=torch.bfloat16))
    assert np.array_equal(ybf, O.bf16_round(y32))


def test_unit_layer_end_to_end(cuda):
    """Unit layer (fp32 X [64, 1024] with 0.5% outliers x50, W [1024, 1024],
    G=256): GPU pack of X and W, GPU linear, against the oracle."""
    wl = config1()
    lin = wl.linears[0]
    x, W, b = wl.X, lin.W, lin.b
    qw_ref, sw_ref, xrw = O.pack(W, 256)
    ref = O.linear(x, qw_ref, sw_ref, b, 256)
    pw = cr.pack_weight(to_dev(W, torch.float32), 256)
    rep_w = R.compare_codes(to_np(pw.q), qw_ref, O.code_values(xrw, sw_ref))
    assert rep_w.ok(), rep_w
    pa = cr.pack_act(to_dev(x, torch.float32), 256)
    rep_x = R.compare_codes(to_np(pa.q), ref["qx"], O.code_values(ref["xrot"], ref["sx"]))
    assert rep_x.ok(), rep_x
    y = to_np(cr.linear(pa, pw, to_dev(b, torch.float32), out_dtype=torch.float32))
    err = R.rel_fro(y, ref["y32"])
    print(f"unit layer: rel Frobenius {err:.3e}; {rep_x}; {rep_w}")
    assert err <= R.Y_RTOL


def test_small_m_kernel_matches_tiled_kernel(cuda):
    K, N = 3072, 1000
    qx, qw = random_codes((48, K), 7), random_codes((N, K), 8)
    s48, sw = np.ones(48, np.float32), np.ones(N, np.float32)
    w = _packed_from_codes(qw, sw, 256, cuda)
    full = cr.linear(_packed_from_codes(qx, s48, 256, cuda), w, out_dtype=torch.int32)
    for m in (1, 5, 16):
        a = _packed_from_codes(qx[:m], s48[:m], 256, cuda)
        small = cr.linear(a, w, out_dtype=torch.int32)
        assert torch.equal(small, full[:m])
        split = cr.linear(a, w, out_dtype=torch.int32, workspace=cr.linear_workspace("plain", m, N, K, cuda))
        assert torch.equal(split, full[:m])


def test_small_m_workspace_is_reusable(cuda):
    """One workspace serves consecutive calls of different shapes (each call
    rewrites what it uses), and a larger one than needed is fine."""
    K = 6912
    big = torch.empty(cr.linear_workspace_bytes("plain", 16, 1152, K) * 2, dtype=torch.uint8, device=cuda)
    for m, n in ((16, 1152), (3, 520), (16, 64)):
        qx, qw = random_codes((m, K), 30 + m), random_codes((n, K), 31 + n)
        a = _packed_from_codes(qx, np.ones(m, np.float32), 256, cuda)
        w = _packed_from_codes(qw, np.ones(n, np.float32), 256, cuda)
        assert cr.linear_workspace_bytes("plain", m, n, K) <= big.numel()
        A = to_np(cr.linear(a, w, out_dtype=torch.int32, workspace=big))
        assert np.array_equal(A.astype(np.int64), O.int_gemm(qx, qw))


def test_row_split_bit_exact(cuda):
    """Rows are independent: 8192-row style chunking (here 256) gives the same bits."""
    x = to_dev(random_rows((700, 1024), 9, dtype="bf16"), torch.bfloat16)
    w = cr.pack_weight(to_dev(random_rows((300, 1024), 10, sigma=0.02, dtype="bf16"), torch.bfloat16), 256)
    b = torch.randn(300, device=cuda) * 0.01
    pa = cr.pack_act(x, 256)
    full = cr.linear(pa, w, b)
    parts = [cr.linear(cr.pack_act(x[s:e], 256), w, b) for s, e in ((0, 256), (256, 512), (512, 700))]
    assert torch.equal(torch.cat(parts), full)
    again = cr.linear(pa, w, b)
    assert torch.equal(again, full)


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (513, 264, 3072), (4096, 1024, 3072), (64, 8, 12288)])
def test_accumulator_matches_vendor_int8_gemm(cuda, M, N, K):
    """The int32 accumulator equals the vendor's int8 GEMM (torch._int_mm on
    hipBLASLt) on the same codes, bit for bit: an integer product has one
    answer."""
    qx = to_dev(random_codes((M, K), seed=M + K), torch.int8)
    qw = to_dev(random_codes((N, K), seed=N + 3 * K), torch.int8)
    try:
        ref = torch._int_mm(qx, qw.t())
    except RuntimeError as e:  # a shape the vendor call does not take
        pytest.skip(f"torch._int_mm: {e}")
    a = cr.Packed(qx, torch.ones(M, device=cuda), 256)
    w = cr.Packed(qw, torch.ones(N, device=cuda), 256)
    assert torch.equal(cr.linear(a, w, out_dtype=torch.int32), ref)


@pytest.mark.parametrize("M", [700, 16])
def test_concatenated_weights_one_launch(cuda, M):
    """Weights are packed row by row, so linears that share one packed
    activation can run as one launch over the concatenated weight: the packed
    concatenation is the concatenation of the packed weights, and each column
    slice of the one output equals that linear's own launch bit for bit."""
    K, G = 1024, 256
    x = to_dev(random_rows((M, K), 21, dtype="bf16"), torch.bfloat16)
    ws = [to_dev(random_rows((n, K), 22 + n, sigma=0.02, dtype="bf16"), torch.bfloat16) for n in (600, 200)]
    bs = [torch.randn(w.shape[0], device=cuda) * 0.01 for w in ws]
    parts = [cr.pack_weight(w, G) for w in ws]
    cat = cr.pack_weight(torch.cat(ws), G)
    assert torch.equal(cat.q, torch.cat([p.q for p in parts]))
    assert torch.equal(cat.scale, torch.cat([p.scale for p in parts]))
    pa = cr.pack_act(x, G)
    y = cr.linear(pa, cat, torch.cat(bs))
    assert torch.equal(y[:, :600], cr.linear(pa, parts[0], bs[0]))
    assert torch.equal(y[:, 600:], cr.linear(pa, parts[1], bs[1]))


def test_strided_output(cuda):
    qx, qw = random_codes((100, 512), 11), random_codes((200, 512), 12)
    a = _packed_from_codes(qx, np.ones(100, np.float32), 256, cuda)
    w = _packed_from_codes(qw, np.ones(200, np.float32), 256, cuda)
    buf = torch.full((100, 264), -7, dtype=torch.int32, device=cuda)
    cr.linear(a, w, out_dtype=torch.int32, out=buf[:, 8:208])
    assert np.array_equal(to_np(buf[:, 8:208]).astype(np.int64), O.int_gemm(qx, qw))
    assert torch.all(buf[:, :8] == -7) and torch.all(buf[:, 208:] == -7)


def test_mismatch_is_an_error(cuda):
    x = to_dev(random_rows((8, 1024), 13, dtype="bf16"), torch.bfloat16)
    w = cr.pack_weight(to_dev(random_rows((16, 1024), 14, dtype="bf16"), torch.bfloat16), 256)
    with pytest.raises(cr.ConvrotError):
        cr.linear(cr.pack_act(x, 64), w)


@pytest.mark.parametrize("M,N,K", [(1, 1152, 6912), (4, 1152, 6912), (12, 1152, 6912), (7, 1000, 4112),
                                   (3, 72, 2048), (12, 4080, 16400), (2, 16, 40960)])
def test_small_m_wide_workgroups(cuda, M, N, K):
    """Up to 12 rows with fewer tiles than CUs: one 16-wave workgroup per tile
    over all of K (staged and register paths, K tails, ragged N); no
    workspace is asked for, and one passed is not used.  Plain, GELU and
    TILE16 weights against the oracle's accumulator; 13 rows take the split."""
    seed = 3 * M + N + K
    qx, qw = random_codes((M, K), seed), random_codes((N, K), seed + 1)
    g = np.random.default_rng(seed)
    sx = g.uniform(0.5, 1.5, M).astype(np.float32) / np.float32(127.0)
    sw = g.uniform(0.5, 1.5, N).astype(np.float32) / np.float32(127.0)
    b = (g.standard_normal(N) * 0.5).astype(np.float32)
    a, w = _packed_from_codes(qx, sx, 16, cuda), _packed_from_codes(qw, sw, 16, cuda)
    assert cr.linear_workspace_bytes("plain", M, N, K) == 0
    A_ref = O.int_gemm(qx, qw)
    assert np.array_equal(to_np(cr.linear(a, w, out_dtype=torch.int32)).astype(np.int64), A_ref)
    spare = torch.empty(1 << 20, dtype=torch.uint8, device=cuda)
    assert np.array_equal(to_np(cr.linear(a, w, out_dtype=torch.int32, workspace=spare)).astype(np.int64), A_ref)
    y64 = O.epilogue64(A_ref, sx, sw, b)
    bd = to_dev(b, torch.float32)
    assert R.rel_fro(to_np(cr.linear(a, w, bd, out_dtype=torch.float32)), y64) <= 1e-5
    y = to_np(cr.linear_act(a, w, bd, cr.GELU_ERF, out_dtype=torch.float32))
    assert R.rel_fro(y, R.gelu64(y64, "gelu_erf")) <= 1e-5
    if N % 16 == 0 and K % 64 == 0:
        t = cr.tile_weight(w)
        assert np.array_equal(to_np(cr.linear(a, t, out_dtype=torch.int32)).astype(np.int64), A_ref)
    # one more row: the K split with its combining launch, the same bits
    qx13 = random_codes((13, K), seed + 2)
    a13 = _packed_from_codes(qx13, np.ones(13, np.float32), 16, cuda)
    ws = cr.linear_workspace("plain", 13, N, K, cuda)
    assert ws is not None or (N + 15) // 16 >= 256 or K < 1024
    A13 = to_np(cr.linear(a13, w, out_dtype=torch.int32, workspace=ws)).astype(np.int64)
    assert np.array_equal(A13, O.int_gemm(qx13, qw))
