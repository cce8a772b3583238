"""convrot_linear_noalloc, the variant of convrot_linear for callers that
cannot allocate: its small-M K split keeps its partial sums in the library's
static per-GPU scratch.  Through the C ABI it must give the same bits as
convrot_linear with a caller workspace, on two calls in a row (the second
with a smaller input, so it runs on scratch the first call left behind), and
the int32 accumulator must equal the oracle's exact product."""

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
from tests.gpu_util import to_dev, to_np
from workloads import random_codes

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed, cuda):
    qx, qw = random_codes((M, K), seed), random_codes((N, K), seed + 1)
    g = np.random.default_rng(seed)
    sx = g.uniform(0.5, 1.5, M).astype(np.float32) / np.float32(127 * 64)
    sw = g.uniform(0.5, 1.5, N).astype(np.float32) / np.float32(127)
    b = (g.standard_normal(N) * 0.01).astype(np.float32)
    a = cr.Packed(to_dev(qx, torch.int8), to_dev(sx, torch.float32), 64)
    w = cr.Packed(to_dev(qw, torch.int8), to_dev(sw, torch.float32), 64)
    return qx, qw, a, w, to_dev(b, torch.float32)


# (M, N, K): the decode down projection (72 tiles, K split 8 ways), then a
# smaller split on the same scratch; then shapes that do not split (432
# tiles; four rows on one 16-wave workgroup per tile), and one on the tiled
# kernel (no scratch at all).
CALLS = [(16, 1152, 6912), (16, 520, 3072), (1, 6912, 1152), (4, 1152, 6912), (40, 300, 1024)]


def test_noalloc_matches_linear_on_consecutive_calls(cuda):
    for i, (M, N, K) in enumerate(CALLS):
        print(f"[noalloc] call {i}: M={M} N={N} K={K}", flush=True)
        qx, qw, a, w, b = _operands(M, N, K, 100 + i, cuda)
        ws = cr.linear_workspace("plain", M, N, K, cuda)
        if i == 0:
            assert ws is not None and ws.numel() <= cr._lib.NOALLOC_SCRATCH_BYTES
        for dt in (torch.int32, torch.bfloat16, torch.float32):
            ref = cr.linear(a, w, None if dt == torch.int32 else b, out_dtype=dt, workspace=ws)
            out = torch.full((M, N), 7, dtype=dt, device=cuda)
            cr.linear_noalloc(a, w, out, None if dt == torch.int32 else b)
            assert torch.equal(out, ref), (i, dt)
            if dt == torch.int32:
                assert np.array_equal(to_np(out).astype(np.int64), O.int_gemm(qx, qw))


def test_noalloc_repeated_call_same_bits(cuda):
    """The scratch keeps the previous call's partials; a call rewrites every
    partial it reads, so repeating a call after a different one changes
    nothing."""
    M, N, K = 16, 1152, 6912
    _, _, a, w, b = _operands(M, N, K, 7, cuda)
    first = cr.linear_noalloc(a, w, torch.empty((M, N), dtype=torch.bfloat16, device=cuda), b)
    _, _, a2, w2, b2 = _operands(16, 900, 4096, 8, cuda)
    cr.linear_noalloc(a2, w2, torch.empty((16, 900), dtype=torch.bfloat16, device=cuda), b2)
    again = cr.linear_noalloc(a, w, torch.empty((M, N), dtype=torch.bfloat16, device=cuda), b)
    assert torch.equal(first, again)
