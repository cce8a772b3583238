"""Parity of the fused rotate + quantise kernel (pack) with the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests import parity as R
from tests.gpu_util import to_dev, to_np
from workloads import random_rows, rademacher, to_bf16_values

pytestmark = pytest.mark.gpu

REGULAR_CASES = [
    # (G, K, M): several groups per row, ragged row counts
    (4, 64, 5), (4, 1040, 3), (16, 1152, 37), (64, 1152, 37), (256, 3072, 37), (256, 1024, 64),
    (256, 12288, 9), (1024, 2048, 11), (1024, 6144, 7), (256, 256, 1), (64, 64, 3), (16, 16, 2),
    (256, 65536, 2),
]


def _inputs(M, K, dtype, seed, outliers=True):
    x = random_rows((M, K), seed, dtype="f32")
    if outliers:
        g = np.random.default_rng(seed + 1)
        pos = g.choice(M * K, size=max(1, M * K // 200), replace=False)
        x.reshape(-1)[pos] *= 50.0
    if dtype == "bf16":
        x = to_bf16_values(x)
    return x


def _check_pack(x, q_gpu, s_gpu, G, kind=O.REGULAR, signs=None):
    q_ref, s_ref, xr_ref = O.pack(x, G, kind, signs)
    v_ref = O.code_values(xr_ref, s_ref)
    rep = R.compare_codes(q_gpu, q_ref, v_ref)
    print(rep)
    assert rep.ok(), rep
    assert R.scale_rel_diff(s_gpu, s_ref) <= R.SCALE_RTOL
    return q_ref, s_ref, xr_ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G,K,M", REGULAR_CASES)
def test_rotate_and_pack_regular(cuda, G, K, M, dtype):
    x = _inputs(M, K, dtype, seed=G * 7 + K + M)
    xd = to_dev(x, torch.bfloat16 if dtype == "bf16" else torch.float32)
    xr_gpu = to_np(cr.rotate(xd, G))
    xr_ref = O.rotate(x, G)
    err = R.rotated_row_err(xr_gpu, xr_ref)
    assert err <= R.ROT_RTOL, err
    p = cr.pack_act(xd, G)
    _check_pack(x, to_np(p.q), to_np(p.scale), G)


@pytest.mark.parametrize("G,K,M", [(128, 1152, 16), (128, 1152, 4), (128, 6912, 5), (16, 1152, 3), (32, 1024, 7),
                                   (64, 2048, 9), (256, 3072, 13), (512, 4096, 3), (1024, 6144, 3)])
def test_rotate_and_pack_randomized(cuda, G, K, M):
    x = _inputs(M, K, "bf16", seed=G + K + M)
    signs = rademacher(5, K)
    xd = to_dev(x, torch.bfloat16)
    sd = to_dev(signs, torch.int8)
    xr_gpu = to_np(cr.rotate(xd, G, cr.RANDOMIZED, sd))
    xr_ref = O.rotate(x, G, O.RANDOMIZED, signs)
    assert R.rotated_row_err(xr_gpu, xr_ref) <= R.ROT_RTOL
    p = cr.pack_act(xd, G, cr.RANDOMIZED, sd)
    _check_pack(x, to_np(p.q), to_np(p.scale), G, O.RANDOMIZED, signs)


def test_pack_weight_equals_pack_act(cuda):
    w = to_dev(random_rows((300, 3072), 5, sigma=0.02, dtype="bf16"), torch.bfloat16)
    a = cr.pack_act(w, 256)
    b = cr.pack_weight(w, 256)
    assert torch.equal(a.q, b.q) and torch.equal(a.scale, b.scale)


def test_zero_constant_and_onehot_rows(cuda):
    K, G = 1024, 256
    x = np.zeros((4, K), dtype=np.float32)
    x[1] = 0.375
    x[2, 300] = -3.0
    x[3, 5] = 2.0
    x[3, 1000] = 1e-3
    p = cr.pack_act(to_dev(x, torch.float32), G)
    q, s = to_np(p.q), to_np(p.scale)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert np.all(q[1] == 127) and s[1] == np.float32(np.float32(0.375) / np.float32(127))
    q_ref, s_ref, _ = O.pack(x, G)
    assert np.array_equal(q[2], q_ref[2]) and s[2] == s_ref[2]
    assert np.all(np.abs(q[2, 256:512]) == 127) and np.all(q[2, :256] == 0) and np.all(q[2, 512:] == 0)
    _check_pack(x, q, s, G)


def test_codes_in_range_and_full_scale(cuda):
    x = _inputs(64, 3072, "bf16", seed=3)
    p = cr.pack_act(to_dev(x, torch.bfloat16), 256)
    q = to_np(p.q)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.max(np.abs(q.astype(np.int16)), axis=1) == 127)


def test_deterministic_and_row_split(cuda):
    x = to_dev(_inputs(600, 3072, "bf16", seed=4), torch.bfloat16)
    a = cr.pack_act(x, 256)
    b = cr.pack_act(x, 256)
    assert torch.equal(a.q, b.q) and torch.equal(a.scale, b.scale)
    parts = [cr.pack_act(x[s:e], 256) for s, e in ((0, 256), (256, 257), (257, 600))]
    assert torch.equal(torch.cat([p.q for p in parts]), a.q)
    assert torch.equal(torch.cat([p.scale for p in parts]), a.scale)


def test_strided_input_and_output(cuda):
    base = to_dev(_inputs(40, 4096, "bf16", seed=6), torch.bfloat16)
    x = base[:, 1024:2048]          # ld 4096, K 1024
    q_buf = torch.zeros((40, 2048), dtype=torch.int8, device=cuda)
    out = cr.Packed(q_buf[:, 512:1536], torch.empty(40, dtype=torch.float32, device=cuda), 256)
    cr.pack_act(x, 256, out=out)
    ref = cr.pack_act(x.contiguous(), 256)
    assert torch.equal(out.q, ref.q) and torch.equal(out.scale, ref.scale)
    assert torch.count_nonzero(q_buf[:, :512]) == 0 and torch.count_nonzero(q_buf[:, 1536:]) == 0
