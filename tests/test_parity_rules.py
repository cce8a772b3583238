"""The comparison rules themselves (CPU only)."""

import numpy as np

from tests import parity as R


def test_codes_accept_flip_at_tie():
    v = np.array([[0.5, 10.49999, 3.2, -7.5]], dtype=np.float32)
    ref = np.array([[0, 10, 3, -8]], dtype=np.int8)
    gpu = np.array([[1, 10, 3, -7]], dtype=np.int8)
    r = R.compare_codes(gpu, ref, v)
    assert r.differ == 2 and r.outside_window == 0 and r.max_abs_diff == 1


def test_codes_reject_flip_away_from_tie():
    v = np.array([[3.2, 1.0]], dtype=np.float32)
    ref = np.array([[3, 1]], dtype=np.int8)
    r = R.compare_codes(np.array([[4, 1]], dtype=np.int8), ref, v)
    assert r.outside_window == 1 and not r.ok()
    r2 = R.compare_codes(np.array([[5, 1]], dtype=np.int8), ref, v)
    assert r2.max_abs_diff == 2 and not r2.ok()


def test_codes_flip_budget():
    n = 100000
    v = np.full((1, n), 0.5, dtype=np.float32)
    ref = np.zeros((1, n), dtype=np.int8)
    gpu = ref.copy()
    gpu[0, :10] = 1
    assert R.compare_codes(gpu, ref, v).ok()
    gpu[0, :11] = 1
    assert not R.compare_codes(gpu, ref, v).ok()


def test_window_widths():
    # 1.27e-4 code units from a tie is inside, 1.3e-4 outside.
    v = np.array([[2.5 + 1.26e-4, 2.5 + 1.3e-4]], dtype=np.float64)
    ref = np.array([[3, 3]], dtype=np.int8)
    gpu = np.array([[2, 2]], dtype=np.int8)
    assert R.compare_codes(gpu, ref, v).outside_window == 1


def test_window_scales_with_code_range():
    # int4 codes (full scale 7): the window is 1e-6 * 7 = 7e-6 code units.
    v = np.array([[2.5 + 6.9e-6, 2.5 + 7.2e-6, 2.5 + 1.2e-4]], dtype=np.float64)
    ref = np.array([[3, 3, 3]], dtype=np.int8)
    gpu = np.array([[2, 2, 2]], dtype=np.int8)
    assert R.compare_codes(gpu, ref, v, qmax=7).outside_window == 2
    assert R.compare_codes(gpu, ref, v).outside_window == 0


def test_scale_and_rows():
    assert R.scale_rel_diff(np.array([1.0, 0.0]), np.array([1.0 + 1e-7, 0.0])) < 1e-6
    assert R.scale_rel_diff(np.array([1.0, 1e-9]), np.array([1.0, 0.0])) == float("inf")
    ref = np.array([[1.0, -2.0], [0.0, 0.0]])
    assert abs(R.rotated_row_err(ref + np.array([[1e-6, 0], [0, 0]]), ref) - 5e-7) < 1e-15
    assert R.rotated_row_err(ref + np.array([[0, 0], [1e-9, 0]]), ref) == float("inf")
    assert abs(R.rel_fro(np.array([3.0, 4.0]) * 1.001, np.array([3.0, 4.0])) - 1e-3) < 1e-12


def test_gelu_reference_matches_torch():
    """The fp64 GELU reference agrees with torch's GELU in both forms."""
    import torch

    y = np.linspace(-8, 8, 4001)
    t = torch.from_numpy(y)
    assert np.max(np.abs(R.gelu64(y, "gelu_erf") - torch.nn.functional.gelu(t).numpy())) < 1e-12
    assert np.max(np.abs(R.gelu64(y, "gelu_tanh") - torch.nn.functional.gelu(t, approximate="tanh").numpy())) < 1e-12
