"""ConvRotLinear: a linear layer on the packed int8 path, with routing.

Routing follows the sglang kitchen_int8 integration (PR 34581 summary page,
implementation section): a layer whose input width K is not a multiple of
the group size stays on the unquantised bf16 linear, and the decision is
logged so that a fallback is never silent.  Non-2-D inputs are flattened to
rows and restored afterwards.
"""

from __future__ import annotations

import logging

import torch

from . import api

log = logging.getLogger("w8a8_int8_linear_amd")


class RoutingLog:
    """Summary of which layers run quantised and which stay in bf16."""

    def __init__(self) -> None:
        self.quantized: list[str] = []
        self.fallback: list[str] = []

    def note(self, name: str, quantized: bool, K: int, G: int) -> None:
        if quantized:
            self.quantized.append(name)
        else:
            self.fallback.append(f"{name}(in={K})")
            log.info("convrot: %s keeps the bf16 linear (K=%d not divisible by G=%d)", name, K, G)

    def summary(self) -> str:
        return (f"convrot: {len(self.quantized)} linear layers int8, {len(self.fallback)} left in bf16"
                + (f": {', '.join(self.fallback)}" if self.fallback else ""))


class ConvRotLinear:
    """Y = X W^T + b through the ConvRot W8A8 path (or the routed bf16 path)."""

    def __init__(self, name: str, N: int, K: int, group: int, kind: str, packed: api.Packed | None,
                 w_bf16: torch.Tensor | None, bias: torch.Tensor | None):
        self.name, self.N, self.K, self.group, self.kind = name, N, K, group, kind
        self.packed = packed
        self.w_bf16 = w_bf16
        self.bias = bias

    @property
    def quantized(self) -> bool:
        return self.packed is not None

    @classmethod
    def from_dense(cls, w: torch.Tensor, bias: torch.Tensor | None = None, group: int = 256,
                   kind: str = api.REGULAR, signs: torch.Tensor | None = None, name: str = "linear",
                   routing: RoutingLog | None = None) -> "ConvRotLinear":
        N, K = w.shape
        b = bias.to(torch.float32).contiguous() if bias is not None else None
        quant = K % group == 0
        if routing is not None:
            routing.note(name, quant, K, group)
        if quant:
            packed = api.pack_weight(w.contiguous(), group, kind, signs)
            return cls(name, N, K, group, kind, packed, None, b)
        return cls(name, N, K, group, kind, None, w.to(torch.bfloat16).contiguous(), b)

    def pack_input(self, x: torch.Tensor) -> api.Packed:
        """Pack rows of x once; reuse the result for every layer with the same
        input and rotation (same group, kind and sign vector)."""
        return api.pack_act(x.reshape(-1, self.K).contiguous(), self.group, self.kind,
                            self.packed.signs if self.packed is not None else None)

    def __call__(self, x: torch.Tensor | api.Packed, out_dtype: torch.dtype | None = None) -> torch.Tensor:
        if isinstance(x, api.Packed):
            if not self.quantized:
                raise ValueError(f"{self.name} is routed to bf16 and cannot take a packed activation")
            return api.linear(x, self.packed, self.bias, out_dtype or torch.bfloat16)
        shape = x.shape
        rows = x.reshape(-1, self.K).contiguous()
        dt = out_dtype or (x.dtype if x.dtype in (torch.float32, torch.bfloat16) else torch.bfloat16)
        if self.quantized:
            y = api.linear(self.pack_input(rows), self.packed, self.bias, dt)
        else:
            y = api.linear_bf16(rows.to(torch.bfloat16), self.w_bf16, self.bias, dt)
        return y.reshape(*shape[:-1], self.N)
