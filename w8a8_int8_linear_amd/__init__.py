"""MI355X-native INT8 ConvRot W8A8 linear layer.

The compute path is libconvrot.so (hand-written HIP for gfx950) behind the C
ABI in include/convrot.h; this package is its Python binding.  Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built.
"""

from .api import (  # noqa: F401
    GELU_ERF, GELU_TANH, PACKIN_MAX_ROWS, RANDOMIZED, REGULAR, ROWS, TILE16, Packed, PackedW4, linear, linear_act,
    linear_act_rowmax, linear_bf16, linear_gated, linear_gated_packin, linear_noalloc, linear_packin, linear_w4,
    linear_w4_gated, linear_workspace, linear_workspace_bytes,
    lora_add, lora_workspace_bytes, pack_act, pack_act_rowmax, pack_weight, pack_weight_w4, rotate, smooth_ffn,
    tile_weight, tile_weight_w4, unpack_w4,
)
from .layer import ConvRotLinear, Route, RoutingLog  # noqa: F401
from ._lib import ConvrotError  # noqa: F401
