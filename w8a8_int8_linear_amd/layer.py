"""ConvRotLinear: a linear layer on the packed int8 path, with routing.

Routing follows the sglang kitchen_int8 integration (PR 34581 summary page,
implementation section): a layer whose input width K is not a multiple of
the group size stays on the unquantised bf16 linear, and the decision is
logged so that a fallback is never silent.  Non-2-D inputs are flattened to
rows and restored afterwards.

Weights are int8 codes, or int4 codes with ``weight_bits=4`` (W4A8, the
int4 ConvRot export of the stable-diffusion.cpp PR "load ConvRot int4 and
per-channel int8 safetensors").  LoRA adapters attached with ``add_lora``
are applied at run time from the unrotated input and added to the base
output ("INT8 Convrot Safetensors", LoRA paragraph); the packed weight is
never modified.
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

    def __init__(self, name: str, N: int, K: int, group: int, kind: str, packed: api.Packed | api.PackedW4 | None,
                 w_bf16: torch.Tensor | None, bias: torch.Tensor | None):
        self.name, self.N, self.K, self.group, self.kind = name, N, K, group, kind
        self.packed = packed
        self.w_bf16 = w_bf16
        self.bias = bias
        self.adapters: list[tuple[torch.Tensor, torch.Tensor, float]] = []

    @property
    def quantized(self) -> bool:
        return self.packed is not None

    @property
    def weight_bits(self) -> int:
        return 4 if isinstance(self.packed, api.PackedW4) else 8

    @classmethod
    def from_dense(cls, w: torch.Tensor, bias: torch.Tensor | None = None, group: int = 256,
                   kind: str = api.REGULAR, signs: torch.Tensor | None = None, name: str = "linear",
                   routing: RoutingLog | None = None, weight_bits: int = 8) -> "ConvRotLinear":
        if weight_bits not in (4, 8):
            raise ValueError("weight_bits must be 8 or 4")
        N, K = w.shape
        b = bias.to(torch.float32).contiguous() if bias is not None else None
        quant = K % group == 0
        if routing is not None:
            routing.note(name, quant, K, group)
        if quant:
            pack = api.pack_weight if weight_bits == 8 else api.pack_weight_w4
            packed = pack(w.contiguous(), group, kind, signs)
            return cls(name, N, K, group, kind, packed, None, b)
        return cls(name, N, K, group, kind, None, w.to(torch.bfloat16).contiguous(), b)

    def add_lora(self, a: torch.Tensor, b: torch.Tensor, scale: float) -> None:
        """Attach an adapter: a [r, K] (down), b [N, r] (up), bf16; its
        correction scale (x a^T) b^T is added to the output at run time."""
        if a.dim() != 2 or b.dim() != 2 or a.shape[1] != self.K or b.shape[0] != self.N or b.shape[1] != a.shape[0]:
            raise ValueError(f"adapter shapes must be a [r, {self.K}] and b [{self.N}, r]")
        self.adapters.append((a.to(torch.bfloat16).contiguous(), b.to(torch.bfloat16).contiguous(), float(scale)))

    def _linear(self, x: api.Packed, dt: torch.dtype) -> torch.Tensor:
        if isinstance(self.packed, api.PackedW4):
            return api.linear_w4(x, self.packed, self.bias, out_dtype=dt)
        return api.linear(x, self.packed, self.bias, dt)

    def pack_input(self, x: torch.Tensor) -> api.Packed:
        """Pack rows of x once; reuse the result for every layer with the same
        input and rotation (same group, kind and sign vector)."""
        return api.pack_act(x.reshape(-1, self.K).contiguous(), self.group, self.kind,
                            self.packed.signs if self.packed is not None else None)

    def __call__(self, x: torch.Tensor | api.Packed, out_dtype: torch.dtype | None = None) -> torch.Tensor:
        if isinstance(x, api.Packed):
            if not self.quantized:
                raise ValueError(f"{self.name} is routed to bf16 and cannot take a packed activation")
            if self.adapters:
                raise ValueError(f"{self.name} has LoRA adapters, which need the unrotated input, not a packed one")
            return self._linear(x, out_dtype or torch.bfloat16)
        shape = x.shape
        rows = x.reshape(-1, self.K).contiguous()
        dt = out_dtype or (x.dtype if x.dtype in (torch.float32, torch.bfloat16) else torch.bfloat16)
        if self.quantized:
            y = self._linear(self.pack_input(rows), dt)
        else:
            y = api.linear_bf16(rows.to(torch.bfloat16), self.w_bf16, self.bias, dt)
        if self.adapters:
            xb = rows.to(torch.bfloat16).contiguous()
            for a, b, scale in self.adapters:
                api.lora_add(xb, a, b, scale, y)
        return y.reshape(*shape[:-1], self.N)
