"""ctypes view of libconvrot.so (the C ABI declared in include/convrot.h).

Loading fails loudly when the library is missing: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libconvrot.so")

ABI_VERSION = 10
NOALLOC_SCRATCH_BYTES = 1 << 20

# convrot_status
OK, ERR_INVALID_ARG, ERR_GROUP, ERR_DTYPE, ERR_ALIGN, ERR_MISMATCH, ERR_HIP = range(7)
# convrot_dtype
F32, BF16, I32 = 0, 1, 2
# convrot_rot_kind
ROT_REGULAR, ROT_RANDOMIZED = 0, 1
# convrot_act
ACT_NONE, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2
# convrot_smooth_norm
SMOOTH_L2, SMOOTH_MAX = 0, 1
# convrot_linear_kind (workspace queries)
LINEAR_PLAIN, LINEAR_GATED, LINEAR_BF16, LINEAR_W4, LINEAR_W4_GATED = range(5)
LAYOUT_ROWS, LAYOUT_TILE16 = 0, 1

EXPORTED = (
    "convrot_pack_act",
    "convrot_pack_weight",
    "convrot_linear",
    "convrot_linear_workspace_bytes",
    "convrot_linear_noalloc",
    "convrot_linear_act",
    "convrot_linear_act_rowmax",
    "convrot_pack_act_rowmax",
    "convrot_linear_gated",
    "convrot_linear_packin",
    "convrot_linear_gated_packin",
    "convrot_linear_bf16",
    "convrot_rotate",
    "convrot_pack_weight_w4",
    "convrot_linear_w4",
    "convrot_linear_w4_gated",
    "convrot_unpack_w4",
    "convrot_tile_weight",
    "convrot_tile_weight_w4",
    "convrot_smooth_ffn",
    "convrot_lora_workspace_bytes",
    "convrot_lora_add",
    "convrot_status_string",
    "convrot_last_error",
    "convrot_abi_version",
)


class Rot(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("kind", ctypes.c_int32), ("signs", ctypes.c_void_p)]


class Packed(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("rot", Rot),
        ("layout", ctypes.c_int32),
    ]


class PackedW4(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("rot", Rot),
        ("layout", ctypes.c_int32),
    ]


class ConvrotError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None
_lock = threading.Lock()


def _declare(lib: ctypes.CDLL) -> None:
    c_int, c_i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    P = ctypes.POINTER(Packed)
    lib.convrot_pack_act.argtypes = [vp, c_int, c_i64, P, vp]
    lib.convrot_pack_act.restype = c_int
    lib.convrot_pack_weight.argtypes = [vp, c_int, c_i64, P, vp]
    lib.convrot_pack_weight.restype = c_int
    lib.convrot_linear.argtypes = [P, P, vp, vp, c_int, c_i64, vp, c_i64, vp]
    lib.convrot_linear.restype = c_int
    lib.convrot_linear_noalloc.argtypes = [P, P, vp, vp, c_int, c_i64, vp]
    lib.convrot_linear_noalloc.restype = c_int
    lib.convrot_linear_workspace_bytes.argtypes = [c_int, c_i64, c_i64, c_i64, ctypes.POINTER(c_i64)]
    lib.convrot_linear_workspace_bytes.restype = c_int
    lib.convrot_linear_act.argtypes = [P, P, vp, c_int, vp, c_int, c_i64, vp, c_i64, vp]
    lib.convrot_linear_act.restype = c_int
    lib.convrot_linear_act_rowmax.argtypes = [P, P, vp, c_int, vp, c_int, c_i64, ctypes.c_int32, vp, c_i64, vp]
    lib.convrot_linear_act_rowmax.restype = c_int
    lib.convrot_pack_act_rowmax.argtypes = [vp, c_int, c_i64, vp, c_i64, P, vp]
    lib.convrot_pack_act_rowmax.restype = c_int
    lib.convrot_linear_gated.argtypes = [P, P, vp, P, vp, c_int, vp, c_int, c_i64, vp, c_i64, vp]
    lib.convrot_linear_gated.restype = c_int
    lib.convrot_linear_packin.argtypes = [vp, c_int, c_i64, c_i64, P, vp, c_int, vp, c_int, c_i64, vp]
    lib.convrot_linear_packin.restype = c_int
    lib.convrot_linear_gated_packin.argtypes = [vp, c_int, c_i64, c_i64, P, vp, P, vp, c_int, vp, c_int, c_i64, vp]
    lib.convrot_linear_gated_packin.restype = c_int
    lib.convrot_linear_bf16.argtypes = [vp, c_i64, vp, c_i64, vp, c_i64, c_i64, c_i64, vp, c_int, c_i64, vp, c_i64,
                                        vp]
    lib.convrot_linear_bf16.restype = c_int
    lib.convrot_rotate.argtypes = [vp, c_int, c_i64, c_i64, c_i64, Rot, vp, c_i64, vp]
    lib.convrot_rotate.restype = c_int
    P4 = ctypes.POINTER(PackedW4)
    lib.convrot_pack_weight_w4.argtypes = [vp, c_int, c_i64, P4, vp]
    lib.convrot_pack_weight_w4.restype = c_int
    lib.convrot_linear_w4.argtypes = [P, P4, vp, c_int, vp, c_int, c_i64, vp, c_i64, vp]
    lib.convrot_linear_w4.restype = c_int
    lib.convrot_linear_w4_gated.argtypes = [P, P4, vp, P4, vp, c_int, vp, c_int, c_i64, vp, c_i64, vp]
    lib.convrot_linear_w4_gated.restype = c_int
    lib.convrot_unpack_w4.argtypes = [P4, vp, c_i64, vp]
    lib.convrot_unpack_w4.restype = c_int
    lib.convrot_tile_weight.argtypes = [ctypes.POINTER(Packed), ctypes.POINTER(Packed), vp]
    lib.convrot_tile_weight.restype = c_int
    lib.convrot_tile_weight_w4.argtypes = [P4, P4, vp]
    lib.convrot_tile_weight_w4.restype = c_int
    lib.convrot_smooth_ffn.argtypes = [vp, c_int, c_i64, vp, c_int, c_i64, c_i64, c_i64, c_i64, c_int, vp, vp, c_i64,
                                       vp, c_i64, vp]
    lib.convrot_smooth_ffn.restype = c_int
    lib.convrot_lora_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.POINTER(c_i64)]
    lib.convrot_lora_workspace_bytes.restype = c_int
    lib.convrot_lora_add.argtypes = [vp, c_i64, c_i64, c_i64, vp, c_i64, vp, c_i64, c_i64, c_i64, ctypes.c_float, vp,
                                     c_int, c_i64, vp, c_i64, vp]
    lib.convrot_lora_add.restype = c_int
    lib.convrot_status_string.argtypes = [c_int]
    lib.convrot_status_string.restype = ctypes.c_char_p
    lib.convrot_last_error.argtypes = []
    lib.convrot_last_error.restype = ctypes.c_char_p
    lib.convrot_abi_version.argtypes = []
    lib.convrot_abi_version.restype = c_int


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libconvrot.so once; raise if it is missing or incompatible."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise ImportError(
                f"{p} is missing: build it with `python -m w8a8_int8_linear_amd.build` "
                "(the library has no fallback path)")
        lib = ctypes.CDLL(p)
        _declare(lib)
        v = lib.convrot_abi_version()
        if v != ABI_VERSION:
            raise ImportError(f"libconvrot ABI {v}, binding expects {ABI_VERSION}")
        if path is None:
            _lib = lib
        return lib


def check(status: int) -> None:
    if status != OK:
        lib = load()
        name = lib.convrot_status_string(status).decode()
        msg = lib.convrot_last_error().decode()
        raise ConvrotError(status, f"{name}: {msg}")
