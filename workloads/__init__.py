"""Seeded synthetic inputs for the ConvRot W8A8 linear workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, quantisation or matmul).  Both the HIP path
and the CPU oracle consume exactly the bits produced here.

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed)`` with
  ``seed = 1000 * config + tensor_id``; tensor ids: X = 1, outlier positions
  = 2, Rademacher signs = 3, weight j = 10 + j, bias j = 20 + j,
  second activation (routed layer) = 4.
* N(0, sigma) means standard deviation sigma.  "p of entries times k" means
  round(p * rows * cols) distinct positions drawn uniformly without
  replacement, multiplied by k.
* bf16 tensors are drawn in fp32 and rounded to bf16 (round-half-to-even, via
  torch's CPU cast); they are returned as fp32 numpy arrays holding exactly
  the bf16 values, plus the dtype tag ``"bf16"``.

The five workloads stand in, by shape and outlier structure only, for the
layers the sources describe (a unit layer, a DiT attention projection, a DiT
MLP pair, a large-M QKV projection with a routed width-2688 layer, and a
gated-FFN decode step).  No real checkpoint or dataset is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

X_ID, POS_ID, SIGN_ID, X2_ID = 1, 2, 3, 4


def _rng(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(1000 * cfg + tensor_id)


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """fp32 array -> fp32 array holding the RNE-rounded bf16 values."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def normal(cfg: int, tensor_id: int, shape, sigma: float) -> np.ndarray:
    g = _rng(cfg, tensor_id)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def scatter_outliers(x: np.ndarray, cfg: int, frac: float, factor: float) -> np.ndarray:
    """Multiply round(frac * x.size) distinct uniform positions by factor."""
    n = int(round(frac * x.size))
    if n:
        pos = _rng(cfg, POS_ID).choice(x.size, size=n, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(factor)
    return x


def column_outliers(x: np.ndarray, cfg: int, ncols: int, factor: float) -> np.ndarray:
    """Multiply ncols seeded columns (every row) by factor."""
    cols = _rng(cfg, POS_ID).choice(x.shape[1], size=ncols, replace=False)
    x[:, cols] *= np.float32(factor)
    return x


def heavy_tail_mixture(cfg: int, shape, p_tail: float, nu: float) -> np.ndarray:
    """N(0,1) entries, each replaced with probability p_tail by Student-t(nu)."""
    g = _rng(cfg, X_ID)
    x = g.standard_normal(size=shape, dtype=np.float32)
    g2 = _rng(cfg, POS_ID)
    mask = g2.random(size=shape, dtype=np.float32) < np.float32(p_tail)
    k = int(mask.sum())
    if k:
        x[mask] = g2.standard_t(nu, size=k).astype(np.float32)
    return x


def rademacher(cfg: int, K: int) -> np.ndarray:
    """Seeded +-1 int8 vector of length K (one sign per input feature)."""
    g = _rng(cfg, SIGN_ID)
    return np.where(g.integers(0, 2, size=K) == 0, 1, -1).astype(np.int8)


@dataclass
class Linear:
    """One linear layer's synthetic operands (weights before packing)."""
    name: str
    W: np.ndarray                # [N, K] fp32 values (bf16-exact when wdtype == "bf16")
    b: np.ndarray | None         # [N] fp32
    wdtype: str


@dataclass
class Workload:
    cfg: int
    name: str
    X: np.ndarray                # [M, K] fp32 values (bf16-exact when xdtype == "bf16")
    xdtype: str
    out_dtype: str
    G: int
    kind: str = "regular"
    signs: np.ndarray | None = None
    linears: list = field(default_factory=list)
    extra: dict = field(default_factory=dict)


def _maybe_bf16(a: np.ndarray, dt: str) -> np.ndarray:
    return to_bf16_values(a) if dt == "bf16" else a


def config1(M: int = 64, K: int = 1024, N: int = 1024) -> Workload:
    """Unit layer: fp32 X ~N(0,1) with 0.5% of entries x50, fp32 W ~N(0,0.02),
    fp32 b ~N(0,0.01), G=256, fp32 output."""
    X = scatter_outliers(normal(1, X_ID, (M, K), 1.0), 1, 0.005, 50.0)
    W = normal(1, 10, (N, K), 0.02)
    b = normal(1, 20, (N,), 0.01)
    return Workload(1, "unit_layer_g256", X, "f32", "f32", 256,
                    linears=[Linear("linear", W, b, "f32")])


def config2(M: int = 4096, K: int = 3072, N_qkv: int = 9216, N_2: int = 3072) -> Workload:
    """DiT attention projection: bf16 X ~N(0,1) with 8 seeded channels x30,
    fused QKV W [9216, 3072] and a second W [3072, 3072] ~N(0,0.02) sharing
    one packed activation, fp32 biases ~N(0,0.01), G=256, bf16 output."""
    X = to_bf16_values(column_outliers(normal(2, X_ID, (M, K), 1.0), 2, 8, 30.0))
    lins = [
        Linear("qkv", to_bf16_values(normal(2, 10, (N_qkv, K), 0.02)), normal(2, 20, (N_qkv,), 0.01), "bf16"),
        Linear("second", to_bf16_values(normal(2, 11, (N_2, K), 0.02)), normal(2, 21, (N_2,), 0.01), "bf16"),
    ]
    return Workload(2, "dit_attn_proj_g256", X, "bf16", "bf16", 256, linears=lins)


def config3(M: int = 8192, K: int = 3072, N_up: int = 12288) -> Workload:
    """DiT MLP pair: bf16 X (N(0,1), 1% Student-t nu=3), W_up [12288, 3072],
    W_down [3072, 12288] ~N(0,0.02), fp32 biases ~N(0,0.01), GELU (erf)
    between the two linears, G=256, bf16 output."""
    X = to_bf16_values(heavy_tail_mixture(3, (M, K), 0.01, 3.0))
    lins = [
        Linear("up", to_bf16_values(normal(3, 10, (N_up, K), 0.02)), normal(3, 20, (N_up,), 0.01), "bf16"),
        Linear("down", to_bf16_values(normal(3, 11, (K, N_up), 0.02)), normal(3, 21, (K,), 0.01), "bf16"),
    ]
    return Workload(3, "dit_mlp_g256", X, "bf16", "bf16", 256, linears=lins,
                    extra={"activation": "gelu_erf"})


def config4(M: int = 32700, K: int = 6144, N: int = 18432,
            K_routed: int = 2688, N_routed: int = 6144, with_routed: bool = True) -> Workload:
    """Large-M QKV: bf16 X ~N(0,1) with 0.1% of entries x100, W [18432, 6144]
    ~N(0,0.015), plus a routed layer X' [M, 2688] -> W' [6144, 2688]
    (2688 % 256 != 0, unquantised bf16 path), G=256, bf16 output."""
    X = to_bf16_values(scatter_outliers(normal(4, X_ID, (M, K), 1.0), 4, 0.001, 100.0))
    lins = [Linear("qkv", to_bf16_values(normal(4, 10, (N, K), 0.015)), normal(4, 20, (N,), 0.01), "bf16")]
    extra = {}
    if with_routed:
        extra["X_routed"] = to_bf16_values(normal(4, X2_ID, (M, K_routed), 1.0))
        extra["routed"] = Linear("adaln_like", to_bf16_values(normal(4, 11, (N_routed, K_routed), 0.02)),
                                 normal(4, 21, (N_routed,), 0.01), "bf16")
    return Workload(4, "large_m_qkv_g256", X, "bf16", "bf16", 256, linears=lins, extra=extra)


def config5(M: int = 16, G: int = 64, kind: str = "regular", K: int = 1152, N: int = 6912) -> Workload:
    """Decode gated FFN: bf16 X [M, 1152] ~N(0,1) with 2 seeded channels x40,
    W_gate, W_up [6912, 1152] sharing one packed activation, W_down
    [1152, 6912], weights ~N(0,0.02), fp32 biases ~N(0,0.01), bf16 output.
    kind == "randomized" draws the seeded +-1 sign vectors (K for gate/up,
    N for down)."""
    X = to_bf16_values(column_outliers(normal(5, X_ID, (M, K), 1.0), 5, 2, 40.0))
    lins = [
        Linear("gate", to_bf16_values(normal(5, 10, (N, K), 0.02)), normal(5, 20, (N,), 0.01), "bf16"),
        Linear("up", to_bf16_values(normal(5, 11, (N, K), 0.02)), normal(5, 21, (N,), 0.01), "bf16"),
        Linear("down", to_bf16_values(normal(5, 12, (K, N), 0.02)), normal(5, 22, (K,), 0.01), "bf16"),
    ]
    signs = rademacher(5, K) if kind == "randomized" else None
    extra = {"signs_down": rademacher(5, N) if kind == "randomized" else None,
             "activation": "gelu_tanh_gated"}
    return Workload(5, f"decode_ffn_m{M}_g{G}{'r' if kind == 'randomized' else ''}", X, "bf16", "bf16", G,
                    kind=kind, signs=signs, linears=lins, extra=extra)


def random_rows(shape, seed: int, sigma: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """Plain seeded N(0, sigma) rows for unit and edge-case tests."""
    x = np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    return _maybe_bf16(x.astype(np.float32), dtype)


def random_codes(shape, seed: int) -> np.ndarray:
    """Seeded int8 codes in [-127, 127], with both extremes forced present."""
    g = np.random.default_rng(seed)
    q = g.integers(-127, 128, size=shape).astype(np.int8)
    if q.size >= 2:
        flat = q.reshape(-1)
        flat[0] = 127
        flat[-1] = -127
    return q


def random_codes4(shape, seed: int) -> np.ndarray:
    """Seeded int4 codes in [-7, 7] (held as int8), with both extremes forced
    present."""
    g = np.random.default_rng(seed)
    q = g.integers(-7, 8, size=shape).astype(np.int8)
    if q.size >= 2:
        flat = q.reshape(-1)
        flat[0] = 7
        flat[-1] = -7
    return q


def smoothing_study_ffn(M: int = 64, K: int = 3072, F: int = 8192, sigma_c: float = 1.5, seed: int = 9):
    """Gated FFN whose intermediate channels are imbalanced: X bf16 [M, K]
    ~N(0,1) with 4 channels x30; W_gate [F, K] ~N(0, 0.02); W_up row j
    ~N(0, 0.02 c_j) and W_down [K, F] column j ~N(0, 0.02 / c_j) with
    c_j = exp(sigma_c z_j), z ~N(0,1).  All bf16 values."""
    g = np.random.default_rng(seed)
    c = np.exp(sigma_c * g.standard_normal(F)).astype(np.float32)
    X = to_bf16_values(column_outliers(g.standard_normal((M, K)).astype(np.float32), seed, 4, 30.0))
    Wg = to_bf16_values((g.standard_normal((F, K)) * 0.02).astype(np.float32))
    Wu = to_bf16_values((g.standard_normal((F, K)) * 0.02 * c[:, None]).astype(np.float32))
    Wd = to_bf16_values((g.standard_normal((K, F)) * 0.02 / c[None, :]).astype(np.float32))
    return X, Wg, Wu, Wd


def lora_adapter(K: int, N: int, r: int, seed: int = 31):
    """Seeded bf16 LoRA pair for a layer [N, K]: A [r, K] ~N(0, 1/K) (down),
    B [N, r] ~N(0, 0.02) (up)."""
    g = np.random.default_rng(seed)
    A = to_bf16_values((g.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32))
    B = to_bf16_values((g.standard_normal((N, r)) * 0.02).astype(np.float32))
    return A, B
