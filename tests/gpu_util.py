"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""

from __future__ import annotations

import numpy as np
import torch


def to_dev(a: np.ndarray, dtype: torch.dtype, device="cuda:0") -> torch.Tensor:
    """Upload an fp32/int array; bf16 targets must already hold bf16 values."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == torch.bfloat16:
        t32 = t.to(torch.float32)
        tb = t32.to(torch.bfloat16)
        assert torch.equal(tb.to(torch.float32), t32), "array is not bf16-exact"
        t = tb
    else:
        t = t.to(dtype)
    return t.to(device)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    torch.cuda.synchronize()
    return t.cpu().numpy()


def dt(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def sample_rows(M: int, seed: int, n_random: int = 64, edge: int = 32) -> np.ndarray:
    """First and last rows, rows around the 256-row tile edges and a seeded
    random set; sorted and unique."""
    g = np.random.default_rng(seed)
    rows = set(range(min(edge, M)))
    rows.update(range(max(0, M - edge), M))
    for t in range(256, M, 256 * max(1, M // 2048)):
        rows.update(r for r in (t - 1, t) if r < M)
    rows.update(g.choice(M, size=min(n_random, M), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
