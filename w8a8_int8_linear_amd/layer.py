"""ConvRotLinear: a linear layer on the packed int8 path, with routing.

Routing follows the sglang kitchen_int8 integration (PR 34581 summary page,
implementation section): a layer whose input width K is not a multiple of
the group size stays on the unquantised bf16 linear.  ``RoutingLog`` keeps
one record per layer (path and reason) and logs every fallback, so that one
is never silent.  Non-2-D inputs are flattened to
rows and restored afterwards.

Weights are int8 codes, or int4 codes with ``weight_bits=4`` (W4A8, the
int4 ConvRot export of the stable-diffusion.cpp PR "load ConvRot int4 and
per-channel int8 safetensors").  LoRA adapters attached with ``add_lora``
are applied at run time from the unrotated input and added to the base
output ("INT8 Convrot Safetensors", LoRA paragraph); the packed weight is
never modified.

Layers that read the same input can share one packed activation (the
stable-diffusion.cpp reuse rule); ``ConvRotLinear.merge`` goes one step
further and runs them as one launch over their stacked packed weights.
Weights are packed row by row, so stacking packed weights equals packing the
stacked weights, and each layer's output is a column slice of the merged
output (``split``).
"""

from __future__ import annotations

import logging
from dataclasses import dataclass

import torch

from . import api

log = logging.getLogger("w8a8_int8_linear_amd")


@dataclass(frozen=True)
class Route:
    """The path one layer takes and why."""
    layer: str
    K: int
    group: int
    path: str     # "int8" or "int4" (quantised ConvRot linear) or "bf16" (unquantised)
    reason: str


class RoutingLog:
    """One ``Route`` per layer built with it.  A layer routed to the
    unquantised bf16 linear is also logged at WARNING level when it is
    recorded, so that a fallback never passes unnoticed."""

    def __init__(self) -> None:
        self.routes: list[Route] = []

    def record(self, layer: str, K: int, group: int, weight_bits: int) -> Route:
        if K % group == 0:
            r = Route(layer, K, group, f"int{weight_bits}", f"G = {group} divides K = {K}")
        else:
            r = Route(layer, K, group, "bf16", f"K = {K} is not a multiple of G = {group}")
            log.warning("convrot: layer %s runs the unquantised bf16 linear (%s)", layer, r.reason)
        self.routes.append(r)
        return r

    def by_path(self, path: str) -> list[Route]:
        return [r for r in self.routes if r.path == path]

    def report(self) -> str:
        """One line per layer: name, input width, path, reason."""
        w = max([len(r.layer) for r in self.routes] + [5])
        lines = [f"{'layer':<{w}}  {'K':>6}  path  reason"]
        lines += [f"{r.layer:<{w}}  {r.K:>6}  {r.path:<4}  {r.reason}" for r in self.routes]
        return "\n".join(lines)


class ConvRotLinear:
    """Y = X W^T + b through the ConvRot W8A8 path (or the routed bf16 path)."""

    def __init__(self, name: str, N: int, K: int, group: int, kind: str, packed: api.Packed | api.PackedW4 | None,
                 w_bf16: torch.Tensor | None, bias: torch.Tensor | None):
        self.name, self.N, self.K, self.group, self.kind = name, N, K, group, kind
        self.packed = packed
        self.w_bf16 = w_bf16
        self.bias = bias
        self.adapters: list[tuple[torch.Tensor, torch.Tensor, float]] = []
        self.splits: list[int] = [N]

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
            routing.record(name, K, group, weight_bits)
        if quant:
            pack = api.pack_weight if weight_bits == 8 else api.pack_weight_w4
            packed = pack(w.contiguous(), group, kind, signs)
            return cls(name, N, K, group, kind, packed, None, b)
        return cls(name, N, K, group, kind, None, w.to(torch.bfloat16).contiguous(), b)

    @classmethod
    def merge(cls, layers: "list[ConvRotLinear]", name: str | None = None) -> "ConvRotLinear":
        """One layer over the stacked packed weights of ``layers``, which must
        all be quantised with the same K, group, rotation (kind and signs) and
        weight width, and carry no adapters.  Its output holds the layers'
        outputs side by side, in order; ``split`` returns them as views."""
        if not layers:
            raise ValueError("merge needs at least one layer")
        first = layers[0]
        for l in layers:
            if not l.quantized:
                raise ValueError(f"{l.name} is routed to bf16 and cannot be merged")
            if l.adapters:
                raise ValueError(f"{l.name} has LoRA adapters; merge the base layers, then attach adapters")
            if (l.K, l.group, l.kind, l.weight_bits) != (first.K, first.group, first.kind, first.weight_bits):
                raise ValueError(f"{l.name} differs from {first.name} in K, group, rotation or weight width")
            s0, s1 = first.packed.signs, l.packed.signs
            if (s0 is None) != (s1 is None) or (s0 is not None and not torch.equal(s0, s1)):
                raise ValueError(f"{l.name} and {first.name} use different sign vectors")
            if l.packed.q.shape[1] != first.packed.q.shape[1]:
                raise ValueError(f"{l.name} and {first.name} have different packed row pitches")
            if l.packed.layout != first.packed.layout:
                raise ValueError(f"{l.name} and {first.name} have different weight layouts")
        q = torch.cat([l.packed.q for l in layers])
        scale = torch.cat([l.packed.scale for l in layers])
        p0 = first.packed
        # (TILE16 weights stack too: each layer's rows are whole 16-row tiles)
        if isinstance(p0, api.PackedW4):
            packed = api.PackedW4(q, scale, p0.K, p0.group, p0.kind, p0.signs, p0.layout)
        else:
            packed = api.Packed(q, scale, p0.group, p0.kind, p0.signs, p0.layout)
        bias = None
        if any(l.bias is not None for l in layers):
            bias = torch.cat([l.bias if l.bias is not None else torch.zeros(l.N, dtype=torch.float32,
                                                                            device=q.device) for l in layers])
        merged = cls(name or "+".join(l.name for l in layers), sum(l.N for l in layers), first.K, first.group,
                     first.kind, packed, None, bias)
        merged.splits = [n for l in layers for n in l.splits]
        return merged

    def tile_for_decode(self) -> None:
        """Keep the packed weight in the TILE16 layout (``api.tile_weight``),
        which the small-M path streams faster; the layer then serves inputs of
        at most 16 rows.  Needs N % 16 == 0 and K % 64 == 0 (int4: K % 128)."""
        if not self.quantized:
            raise ValueError(f"{self.name} is routed to bf16; only packed weights are tiled")
        tile = api.tile_weight_w4 if isinstance(self.packed, api.PackedW4) else api.tile_weight
        self.packed = tile(self.packed)

    def split(self, y: torch.Tensor) -> tuple[torch.Tensor, ...]:
        """The outputs of the layers a merged layer was made from, as column
        views of its output y."""
        return torch.split(y, self.splits, dim=-1)

    def add_lora(self, a: torch.Tensor, b: torch.Tensor, scale: float) -> None:
        """Attach an adapter: a [r, K] (down), b [N, r] (up), bf16; its
        correction scale (x a^T) b^T is added to the output at run time."""
        if a.dim() != 2 or b.dim() != 2 or a.shape[1] != self.K or b.shape[0] != self.N or b.shape[1] != a.shape[0]:
            raise ValueError(f"adapter shapes must be a [r, {self.K}] and b [{self.N}, r]")
        self.adapters.append((a.to(torch.bfloat16).contiguous(), b.to(torch.bfloat16).contiguous(), float(scale)))

    def _workspace(self, kind: str, M: int, device: torch.device) -> torch.Tensor | None:
        """The split-K workspace of a small-M call (a torch allocation of the
        caller's; None when the shape does not split).  Above 16 rows the
        int4 binding allocates its expanded-weight workspace itself."""
        return api.linear_workspace(kind, M, self.N, self.K, device) if M <= 16 else None

    def _linear(self, x: api.Packed, dt: torch.dtype) -> torch.Tensor:
        if isinstance(self.packed, api.PackedW4):
            return api.linear_w4(x, self.packed, self.bias, out_dtype=dt,
                                 workspace=self._workspace(api.W4, x.rows, x.q.device))
        return api.linear(x, self.packed, self.bias, dt, workspace=self._workspace(api.PLAIN, x.rows, x.q.device))

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
            y = api.linear_bf16(rows.to(torch.bfloat16), self.w_bf16, self.bias, dt,
                                workspace=self._workspace(api.BF16, rows.shape[0], rows.device))
        if self.adapters:
            xb = rows.to(torch.bfloat16).contiguous()
            for a, b, scale in self.adapters:
                api.lora_add(xb, a, b, scale, y)
        return y.reshape(*shape[:-1], self.N)
