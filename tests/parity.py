"""Comparison rules between the HIP path and the CPU oracle.

Readings of the tolerances (see the design notes):

* Codes (Q_x, Q_w): a GPU code may differ from the oracle's by exactly 1,
  and only where the oracle's fp32 code value v lies within
  TIE_REL * qmax of a rounding tie, i.e. within 1e-6 of the row's
  full-scale code (qmax = 127 for int8: 1.27e-4 code units; qmax = 7 for
  int4 weights: 7e-6 code units); at most FLIP_FRAC of all elements may
  differ.  The count under the stricter reading (|v - tie| <= 1e-6 |v|) is
  reported as well.
* Scales: relative difference <= 1e-5.
* Rotated fp32 rows: per row, max |diff| <= 1e-5 * max |oracle row|.
* The int32 accumulator: bit-exact.
* fp32 Y: relative Frobenius error <= 2e-3 against the oracle's fp32 Y;
  bf16 Y against the bf16 rounding of the oracle's fp32 Y, same bound.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TIE_REL = 1e-6
FLIP_FRAC = 1e-4
SCALE_RTOL = 1e-5
ROT_RTOL = 1e-5
Y_RTOL = 2e-3


@dataclass
class CodeReport:
    n: int
    differ: int
    max_abs_diff: int
    outside_window: int
    strict_outside: int

    def ok(self) -> bool:
        return (self.max_abs_diff <= 1 and self.outside_window == 0
                and self.differ <= max(FLIP_FRAC * self.n, 0))

    def __str__(self) -> str:
        return (f"codes: {self.differ}/{self.n} differ (max |d| {self.max_abs_diff}), "
                f"{self.outside_window} outside the tie window, {self.strict_outside} outside the strict window")


def compare_codes(q_gpu: np.ndarray, q_ref: np.ndarray, v_ref: np.ndarray, qmax: int = 127) -> CodeReport:
    q_gpu = np.asarray(q_gpu).astype(np.int16)
    q_ref = np.asarray(q_ref).astype(np.int16)
    d = q_gpu - q_ref
    idx = np.nonzero(d)
    v = np.asarray(v_ref, np.float64)[idx]
    tie_dist = np.abs(v - (np.floor(v) + 0.5))
    outside = int(np.count_nonzero(tie_dist > TIE_REL * qmax))
    strict = int(np.count_nonzero(tie_dist > TIE_REL * np.abs(v)))
    return CodeReport(int(q_ref.size), int(idx[0].size), int(np.max(np.abs(d))) if d.size else 0, outside, strict)


def scale_rel_diff(s_gpu: np.ndarray, s_ref: np.ndarray) -> float:
    s_gpu = np.asarray(s_gpu, np.float64)
    s_ref = np.asarray(s_ref, np.float64)
    den = np.where(s_ref == 0, 1.0, np.abs(s_ref))
    bad_zero = np.any((s_ref == 0) != (s_gpu == 0))
    return float("inf") if bad_zero else float(np.max(np.abs(s_gpu - s_ref) / den)) if s_ref.size else 0.0


def rotated_row_err(r_gpu: np.ndarray, r_ref: np.ndarray) -> float:
    """max over rows of max|diff| / max|ref row| (0-rows must match exactly)."""
    r_gpu = np.asarray(r_gpu, np.float64)
    r_ref = np.asarray(r_ref, np.float64)
    num = np.max(np.abs(r_gpu - r_ref), axis=1)
    den = np.max(np.abs(r_ref), axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(np.max(out)) if out.size else 0.0


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))


def gelu64(y: np.ndarray, act: str) -> np.ndarray:
    """GELU in fp64 from its definition: act "gelu_erf" is y/2 (1 + erf(y/sqrt 2)),
    "gelu_tanh" is y/2 (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).  The
    activation after a linear layer, not part of the method."""
    from scipy.special import erf

    y = np.asarray(y, np.float64)
    if act == "gelu_erf":
        return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))
    if act == "gelu_tanh":
        return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))
    raise ValueError(act)
