"""MI355X-native INT8 ConvRot W8A8 linear layer.

The compute path is libconvrot.so (hand-written HIP for gfx950) behind the C
ABI in include/convrot.h; this package is its Python binding.  Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built.
"""

from .api import (  # noqa: F401
    GELU_ERF, GELU_TANH, RANDOMIZED, REGULAR, Packed, linear, linear_act, linear_bf16, linear_gated, pack_act,
    pack_weight, rotate,
)
from .layer import ConvRotLinear, RoutingLog  # noqa: F401
from ._lib import ConvrotError  # noqa: F401
