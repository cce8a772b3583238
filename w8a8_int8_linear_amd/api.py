"""Python binding of the ConvRot W8A8 linear C ABI.

Every function marshals torch CUDA tensors (device memory) and the current
torch stream into a call of libconvrot.so; all arithmetic happens in the HIP
kernels.  Shapes, dtypes, strides and devices of caller-supplied outputs are
checked here before any call, since the library takes sizes from the
operands.  Names follow the C entry points: ``pack_act``, ``pack_weight``,
``linear``, ``linear_act``, ``linear_gated``, ``linear_bf16``, ``rotate``,
for int4 weights (W4A8) ``pack_weight_w4``, ``linear_w4``,
``linear_w4_gated``, ``unpack_w4``, the offline ``smooth_ffn`` and the
runtime adapter correction ``lora_add``.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

REGULAR = "regular"
RANDOMIZED = "randomized"
_KIND = {REGULAR: _lib.ROT_REGULAR, RANDOMIZED: _lib.ROT_RANDOMIZED}
_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16, torch.int32: _lib.I32}
ROWS = "rows"
TILE16 = "tile16"
_LAYOUT = {ROWS: _lib.LAYOUT_ROWS, TILE16: _lib.LAYOUT_TILE16}
GELU_ERF = "gelu_erf"
GELU_TANH = "gelu_tanh"
_ACT = {GELU_ERF: _lib.ACT_GELU_ERF, GELU_TANH: _lib.ACT_GELU_TANH}


@dataclass
class Packed:
    """int8 rows + one fp32 scale per row + the rotation that produced them.

    Used both for a packed activation (rows = tokens) and for a packed weight
    (rows = output features).  ``signs`` (int8 +-1, length K) is kept alive
    with the codes because the rotation descriptor points at it.
    """
    q: torch.Tensor          # [rows, K] int8 (row stride may exceed K)
    scale: torch.Tensor      # [rows] fp32
    group: int
    kind: str = REGULAR
    signs: torch.Tensor | None = None
    layout: str = ROWS       # ROWS, or TILE16 for operands read only at M <= 16 (tile_weight, pack_act)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def K(self) -> int:
        return self.q.shape[1]

    def descriptor(self) -> _lib.Packed:
        q, s = self.q, self.scale
        if q.dtype != torch.int8 or q.dim() != 2:
            raise ValueError("packed codes must be a 2-D int8 tensor")
        if q.shape[1] > 1 and q.stride(1) != 1:
            raise ValueError("packed codes must have unit stride along K")
        if s.dtype != torch.float32 or s.dim() != 1 or s.numel() != q.shape[0] or not s.is_contiguous():
            raise ValueError("packed scales must be a contiguous float32 vector with one entry per row")
        if not q.is_cuda or s.device != q.device:
            raise ValueError("packed codes and scales must be device tensors on one device")
        return _lib.Packed(q.data_ptr(), s.data_ptr(), q.shape[0], q.shape[1], _ld(q),
                           _rot(self.group, self.kind, self.signs), _layout(self.layout))


def _layout(layout: str) -> int:
    if layout not in _LAYOUT:
        raise ValueError(f"layout must be one of {sorted(_LAYOUT)}, got {layout!r}")
    return _LAYOUT[layout]


def _rot(group: int, kind: str, signs: torch.Tensor | None) -> _lib.Rot:
    if kind not in _KIND:
        raise ValueError(f"unknown rotation kind {kind!r}")
    return _lib.Rot(int(group), _KIND[kind], signs.data_ptr() if signs is not None else None)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_cuda(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2 or (t.shape[0] > 1 and t.stride(1) != 1) or (t.shape[0] <= 1 and t.numel() and t.stride(-1) != 1):
        raise ValueError(f"{name} must be 2-D with unit stride along K")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _check_out(out: torch.Tensor, M: int, N: int, dtypes, device: torch.device) -> None:
    """A caller's output must be exactly [M, N] with unit column stride on
    the operands' device: the library takes M and N from the operands and
    only the row pitch from ``out``, so anything smaller would be written
    past its end."""
    if out.dtype not in dtypes:
        raise ValueError(f"output dtype must be one of {[str(d) for d in dtypes]}, got {out.dtype}")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"output must have shape [{M}, {N}], got {list(out.shape)}")
    if N > 1 and out.stride(1) != 1:
        raise ValueError("output must have unit stride along its columns")
    if M > 1 and out.stride(0) < N:
        raise ValueError("output rows overlap (row stride below N)")
    if out.device != device:
        raise ValueError(f"output is on {out.device}, the operands on {device}")


def _check_bias(bias: torch.Tensor | None, N: int, device: torch.device, name: str = "bias") -> None:
    if bias is None:
        return
    if bias.dtype != torch.float32 or bias.numel() != N or not bias.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 vector of length N")
    if bias.device != device:
        raise ValueError(f"{name} is on {bias.device}, the operands on {device}")


def _ptr(t: torch.Tensor | None):
    return t.data_ptr() if t is not None else None


# ---------------------------------------------------------------------------
# Workspaces of the linear entry points
# ---------------------------------------------------------------------------

PLAIN, GATED, BF16, W4, W4_GATED = "plain", "gated", "bf16", "w4", "w4_gated"
_LINEAR_KIND = {PLAIN: _lib.LINEAR_PLAIN, GATED: _lib.LINEAR_GATED, BF16: _lib.LINEAR_BF16, W4: _lib.LINEAR_W4,
                W4_GATED: _lib.LINEAR_W4_GATED}


def linear_workspace_bytes(kind: str, M: int, N: int, K: int) -> int:
    """Bytes of workspace a linear call of ``kind`` ("plain" for linear and
    linear_act, "gated", "bf16", "w4", "w4_gated") uses for X [M, K] and N
    outputs on the current device (convrot_linear_workspace_bytes).  With
    M <= 16 it is the optional split-K partial-sum buffer (0 when the shape
    does not split); with M > 16 only the int4 kinds need one."""
    if kind not in _LINEAR_KIND:
        raise ValueError(f"kind must be one of {sorted(_LINEAR_KIND)}")
    lib = _lib.load()
    out = ctypes.c_int64(0)
    _lib.check(lib.convrot_linear_workspace_bytes(_LINEAR_KIND[kind], M, N, K, ctypes.byref(out)))
    return out.value


def linear_workspace(kind: str, M: int, N: int, K: int, device: torch.device) -> torch.Tensor | None:
    """A device buffer of ``linear_workspace_bytes(kind, M, N, K)`` bytes,
    or None when that is 0 (a caller-side convenience: the buffer is an
    ordinary torch allocation owned by the caller)."""
    with torch.cuda.device(device):
        n = linear_workspace_bytes(kind, M, N, K)
    return torch.empty((n,), dtype=torch.uint8, device=device) if n else None


def _ws(workspace: torch.Tensor | None, device: torch.device):
    """(pointer, bytes) of an optional workspace tensor."""
    if workspace is None:
        return None, 0
    if not workspace.is_contiguous() or workspace.device != device:
        raise ValueError("workspace must be a contiguous tensor on the operands' device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _check_signs(signs, K, kind):
    if kind == RANDOMIZED:
        if signs is None:
            raise ValueError("the randomized rotation needs a sign vector")
        if signs.dtype != torch.int8 or signs.numel() != K or not signs.is_cuda or not signs.is_contiguous():
            raise ValueError("signs must be a contiguous int8 device vector of length K")
    elif signs is not None:
        raise ValueError("signs are only used by the randomized rotation")


def _pack(fn, x: torch.Tensor, group: int, kind: str, signs, out: Packed | None, layout: str = ROWS) -> Packed:
    _need_cuda(x, "input")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("input must be float32 or bfloat16")
    rows, K = x.shape
    _check_signs(signs, K, kind)
    if out is None:
        _layout(layout)
        if layout == TILE16 and (rows > 16 or K % 64):
            raise ValueError("a TILE16 activation needs M <= 16 and K % 64 == 0")
        # a TILE16 activation is one 16-row tile (16 * K bytes) whatever M is
        q = torch.empty((16 if layout == TILE16 else rows, K), dtype=torch.int8, device=x.device)[:rows]
        out = Packed(q, torch.empty((rows,), dtype=torch.float32, device=x.device), group, kind, signs, layout)
    desc = out.descriptor()
    _lib.check(fn(x.data_ptr(), _DT[x.dtype], _ld(x), ctypes.byref(desc), _stream(x.device)))
    return out


def pack_act(x: torch.Tensor, group: int = 256, kind: str = REGULAR, signs: torch.Tensor | None = None,
             out: Packed | None = None, layout: str = ROWS) -> Packed:
    """Rotate + quantise activation rows (convrot_pack_act).  ``layout=TILE16``
    (M <= 16, K % 64 == 0) writes the codes as one 16-row tile whose 64-byte
    K units are each 1 KiB of consecutive memory, the layout the small-M
    kernel reads in whole cache lines; only the int8-weight linear, act and
    gated calls accept such an activation.  ``out`` keeps its own layout."""
    return _pack(_lib.load().convrot_pack_act, x, group, kind, signs, out, layout)


def pack_weight(w: torch.Tensor, group: int = 256, kind: str = REGULAR, signs: torch.Tensor | None = None,
                out: Packed | None = None) -> Packed:
    """Rotate + quantise weight rows offline (convrot_pack_weight)."""
    return _pack(_lib.load().convrot_pack_weight, w, group, kind, signs, out)


def linear(act: Packed, w: Packed, bias: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = A * s_x * s_w + b from a packed activation and a packed weight
    (convrot_linear).  ``out_dtype=torch.int32`` returns the raw accumulator.
    ``workspace`` (see ``linear_workspace``) lets M <= 16 split K across
    workgroups; without one the unsplit kernel runs (same result bits)."""
    M, N = act.rows, w.rows
    dev = act.q.device
    if out is None:
        if out_dtype not in _DT:
            raise ValueError("output must be float32, bfloat16 or int32")
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _check_out(out, M, N, tuple(_DT), dev)
    _check_bias(bias, N, dev)
    a, b = act.descriptor(), w.descriptor()
    wp, wn = _ws(workspace, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear(ctypes.byref(a), ctypes.byref(b), _ptr(bias), out.data_ptr(), _DT[out.dtype],
                                  _ld(out), wp, wn, _stream(dev)))
    return out


def linear_noalloc(act: Packed, w: Packed, out: torch.Tensor, bias: torch.Tensor | None = None) -> torch.Tensor:
    """``linear`` for callers that cannot allocate (convrot_linear_noalloc):
    the caller passes ``out`` [M, N] (float32, bfloat16 or int32); the
    small-M split's partial sums go to the library's static per-GPU scratch.
    Calls that overlap in time on one GPU race on that scratch."""
    M, N = act.rows, w.rows
    dev = act.q.device
    _check_out(out, M, N, tuple(_DT), dev)
    _check_bias(bias, N, dev)
    a, b = act.descriptor(), w.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_linear_noalloc(ctypes.byref(a), ctypes.byref(b), _ptr(bias), out.data_ptr(),
                                          _DT[out.dtype], _ld(out), _stream(dev)))
    return out


def _out_and_bias(M, N, device, out, out_dtype, bias):
    if out is None:
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("output must be float32 or bfloat16")
        out = torch.empty((M, N), dtype=out_dtype, device=device)
    _check_out(out, M, N, (torch.float32, torch.bfloat16), device)
    _check_bias(bias, N, device)
    return out


def _act_code(act: str) -> int:
    if act not in _ACT:
        raise ValueError(f"activation must be one of {sorted(_ACT)}")
    return _ACT[act]


def linear_act(act_in: Packed, w: Packed, bias: torch.Tensor | None = None, act: str = GELU_ERF,
               out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = act(A * s_x * s_w + b) with the activation in the epilogue
    (convrot_linear_act); ``workspace`` as in ``linear``."""
    dev = act_in.q.device
    out = _out_and_bias(act_in.rows, w.rows, dev, out, out_dtype, bias)
    a, b = act_in.descriptor(), w.descriptor()
    wp, wn = _ws(workspace, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear_act(ctypes.byref(a), ctypes.byref(b), _ptr(bias), _act_code(act), out.data_ptr(),
                                      _DT[out.dtype], _ld(out), wp, wn, _stream(dev)))
    return out


def linear_act_rowmax(act_in: Packed, w: Packed, group_next: int = 256, bias: torch.Tensor | None = None,
                      act: str = GELU_ERF, out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      rowmax: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """``linear_act`` that also returns, for the layer reading its output,
    the largest magnitude of every group of ``group_next`` output features
    after the regular rotation (convrot_linear_act_rowmax): (Y, rowmax
    [M, N / group_next]).  ``pack_act_rowmax(Y, rowmax, group_next)`` then
    equals ``pack_act(Y, group_next)`` bit for bit."""
    dev = act_in.q.device
    M, N = act_in.rows, w.rows
    out = _out_and_bias(M, N, dev, out, out_dtype, bias)
    if group_next <= 0 or N % group_next:
        raise ValueError("group_next must divide N")
    if rowmax is None:
        rowmax = torch.empty((M, N // group_next), dtype=torch.float32, device=dev)
    if rowmax.dtype != torch.float32 or tuple(rowmax.shape) != (M, N // group_next) or rowmax.device != dev or \
            (rowmax.shape[1] > 1 and rowmax.stride(1) != 1):
        raise ValueError(f"rowmax must be float32 [{M}, {N // group_next}] on the operands' device")
    a, b = act_in.descriptor(), w.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_linear_act_rowmax(ctypes.byref(a), ctypes.byref(b), _ptr(bias), _act_code(act),
                                             out.data_ptr(), _DT[out.dtype], _ld(out), int(group_next),
                                             rowmax.data_ptr(), _ld(rowmax), _stream(dev)))
    return out, rowmax


def pack_act_rowmax(x: torch.Tensor, rowmax: torch.Tensor, group: int = 256, out: Packed | None = None) -> Packed:
    """Pack rows of x whose rotated group maxima are given (from
    ``linear_act_rowmax``) without reducing the rows again
    (convrot_pack_act_rowmax); regular rotation only."""
    _need_cuda(x, "input")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("input must be float32 or bfloat16")
    rows, K = x.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide K")
    if rowmax.dtype != torch.float32 or tuple(rowmax.shape) != (rows, K // group) or rowmax.device != x.device or \
            (rowmax.shape[1] > 1 and rowmax.stride(1) != 1):
        raise ValueError(f"rowmax must be float32 [{rows}, {K // group}] on the input's device")
    if out is None:
        out = Packed(torch.empty((rows, K), dtype=torch.int8, device=x.device),
                     torch.empty((rows,), dtype=torch.float32, device=x.device), group)
    desc = out.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_pack_act_rowmax(x.data_ptr(), _DT[x.dtype], _ld(x), rowmax.data_ptr(), _ld(rowmax),
                                           ctypes.byref(desc), _stream(x.device)))
    return out


def linear_gated(act_in: Packed, w_gate: Packed, w_up: Packed, b_gate: torch.Tensor | None = None,
                 b_up: torch.Tensor | None = None, act: str = GELU_TANH, out_dtype: torch.dtype = torch.bfloat16,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = act(gate) * up for two weights sharing one packed activation, in
    one launch (convrot_linear_gated); ``workspace`` as in ``linear`` (kind
    "gated")."""
    dev = act_in.q.device
    out = _out_and_bias(act_in.rows, w_gate.rows, dev, out, out_dtype, b_gate)
    _check_bias(b_up, w_up.rows, dev, "b_up")
    a, g, u = act_in.descriptor(), w_gate.descriptor(), w_up.descriptor()
    wp, wn = _ws(workspace, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear_gated(
        ctypes.byref(a), ctypes.byref(g), _ptr(b_gate), ctypes.byref(u), _ptr(b_up), _act_code(act),
        out.data_ptr(), _DT[out.dtype], _ld(out), wp, wn, _stream(dev)))
    return out


PACKIN_MAX_ROWS = 4


def _packin_input(x: torch.Tensor, w: Packed) -> None:
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be a bfloat16 [M, {w.K}] tensor")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("x must have unit stride along K")
    if x.device != w.q.device:
        raise ValueError("x and the packed weight must be on one device")


def linear_packin(x: torch.Tensor, w: Packed, bias: torch.Tensor | None = None, act: str | None = None,
                  out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """``linear`` (or ``linear_act`` with ``act``) of bf16 rows x [M, K],
    M <= PACKIN_MAX_ROWS, packed inside the same launch with the weight's
    rotation (convrot_linear_packin): the result bits of
    ``linear(pack_act(x, ...), w)`` in one launch instead of two."""
    _packin_input(x, w)
    M, N = x.shape[0], w.rows
    dev = x.device
    if act is None:
        if out is None:
            if out_dtype not in _DT:
                raise ValueError("output must be float32, bfloat16 or int32")
            out = torch.empty((M, N), dtype=out_dtype, device=dev)
        _check_out(out, M, N, tuple(_DT), dev)
        _check_bias(bias, N, dev)
        code = _lib.ACT_NONE
    else:
        out = _out_and_bias(M, N, dev, out, out_dtype, bias)
        code = _act_code(act)
    b = w.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_linear_packin(x.data_ptr(), _lib.BF16, _ld(x), M, ctypes.byref(b), _ptr(bias), code,
                                         out.data_ptr(), _DT[out.dtype], _ld(out), _stream(dev)))
    return out


def linear_gated_packin(x: torch.Tensor, w_gate: Packed, w_up: Packed, b_gate: torch.Tensor | None = None,
                        b_up: torch.Tensor | None = None, act: str = GELU_TANH,
                        out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """``linear_gated`` of bf16 rows x [M, K], M <= PACKIN_MAX_ROWS, packed
    inside the same launch (convrot_linear_gated_packin)."""
    _packin_input(x, w_gate)
    M = x.shape[0]
    dev = x.device
    out = _out_and_bias(M, w_gate.rows, dev, out, out_dtype, b_gate)
    _check_bias(b_up, w_up.rows, dev, "b_up")
    g, u = w_gate.descriptor(), w_up.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_linear_gated_packin(
        x.data_ptr(), _lib.BF16, _ld(x), M, ctypes.byref(g), _ptr(b_gate), ctypes.byref(u), _ptr(b_up),
        _act_code(act), out.data_ptr(), _DT[out.dtype], _ld(out), _stream(dev)))
    return out


def linear_bf16(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
                out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Unquantised bf16 linear Y = X W^T + b for routed layers
    (convrot_linear_bf16); ``workspace`` as in ``linear`` (kind "bf16")."""
    if x.dim() != 2 or w.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bfloat16")
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    out = _out_and_bias(M, N, dev, out, out_dtype, bias)
    _need_cuda(x, "x")
    _need_cuda(w, "w")
    if w.device != dev:
        raise ValueError("x and w must be on one device")
    wp, wn = _ws(workspace, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear_bf16(x.data_ptr(), _ld(x), w.data_ptr(), _ld(w), _ptr(bias), M, N, K,
                                       out.data_ptr(), _DT[out.dtype], _ld(out), wp, wn, _stream(dev)))
    return out


def rotate(x: torch.Tensor, group: int = 256, kind: str = REGULAR, signs: torch.Tensor | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 rotated rows X R from the pack kernel with quantisation off (convrot_rotate)."""
    _need_cuda(x, "x")
    M, K = x.shape
    _check_signs(signs, K, kind)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=x.device)
    lib = _lib.load()
    _lib.check(lib.convrot_rotate(x.data_ptr(), _DT[x.dtype], M, K, _ld(x), _rot(group, kind, signs),
                                  out.data_ptr(), _ld(out), _stream(x.device)))
    return out


# ---------------------------------------------------------------------------
# int4 weights (W4A8)
# ---------------------------------------------------------------------------

@dataclass
class PackedW4:
    """int4 weight: nibble pairs (element 2j in the low nibble of byte j),
    one fp32 scale per output row (row max / 7), and the rotation."""
    q: torch.Tensor          # [rows, K / 2] uint8 (row stride may exceed K / 2)
    scale: torch.Tensor      # [rows] fp32
    K: int
    group: int
    kind: str = REGULAR
    signs: torch.Tensor | None = None
    layout: str = ROWS       # ROWS, or TILE16 (tile_weight_w4)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    def descriptor(self) -> _lib.PackedW4:
        q, s = self.q, self.scale
        if q.dtype != torch.uint8 or q.dim() != 2 or q.shape[1] * 2 != self.K:
            raise ValueError("q must be uint8 [rows, K / 2]")
        if q.shape[1] > 1 and q.stride(1) != 1:
            raise ValueError("q must have unit stride along its bytes")
        if s.dtype != torch.float32 or s.dim() != 1 or s.numel() != q.shape[0] or not s.is_contiguous():
            raise ValueError("scales must be a contiguous float32 vector with one entry per row")
        if not q.is_cuda or s.device != q.device:
            raise ValueError("q and scales must be device tensors on one device")
        return _lib.PackedW4(self.q.data_ptr(), self.scale.data_ptr(), self.q.shape[0], self.K, _ld(self.q),
                             _rot(self.group, self.kind, self.signs), _layout(self.layout))


def pack_weight_w4(w: torch.Tensor, group: int = 256, kind: str = REGULAR, signs: torch.Tensor | None = None,
                   out: PackedW4 | None = None) -> PackedW4:
    """Rotate, quantise to int4 and pack weight rows offline (convrot_pack_weight_w4)."""
    _need_cuda(w, "w")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    rows, K = w.shape
    _check_signs(signs, K, kind)
    if out is None:
        out = PackedW4(torch.empty((rows, K // 2), dtype=torch.uint8, device=w.device),
                       torch.empty((rows,), dtype=torch.float32, device=w.device), K, group, kind, signs)
    desc = out.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_pack_weight_w4(w.data_ptr(), _DT[w.dtype], _ld(w), ctypes.byref(desc), _stream(w.device)))
    return out


def _w4_workspace(kind: str, M: int, N: int, K: int, device, workspace):
    """The workspace of an int4 call: required above 16 rows (allocated here
    when not given), optional at or below."""
    if M <= 16 or workspace is not None:
        return workspace
    return linear_workspace(kind, M, N, K, device)


def linear_w4(act_in: Packed, w: PackedW4, bias: torch.Tensor | None = None, act: str | None = None,
              out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8 linear Y = act(A * s_x * s_w + b), act None for the plain linear
    (convrot_linear_w4).  For more than 16 rows the expanded int8 weight goes
    to ``workspace`` (allocated here when not given); at or below 16 rows a
    workspace is optional and enables the K split, as in ``linear``."""
    M, N = act_in.rows, w.rows
    dev = act_in.q.device
    if out is None:
        if out_dtype not in _DT:
            raise ValueError("output must be float32, bfloat16 or int32")
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _check_out(out, M, N, tuple(_DT) if act is None else (torch.float32, torch.bfloat16), dev)
    _check_bias(bias, N, dev)
    ws = _w4_workspace(W4, M, N, w.K, dev, workspace)
    a, b = act_in.descriptor(), w.descriptor()
    wp, wn = _ws(ws, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear_w4(ctypes.byref(a), ctypes.byref(b), _ptr(bias),
                                     _lib.ACT_NONE if act is None else _act_code(act), out.data_ptr(), _DT[out.dtype],
                                     _ld(out), wp, wn, _stream(dev)))
    return out


def linear_w4_gated(act_in: Packed, w_gate: PackedW4, w_up: PackedW4, b_gate: torch.Tensor | None = None,
                    b_up: torch.Tensor | None = None, act: str = GELU_TANH, out_dtype: torch.dtype = torch.bfloat16,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = act(gate) * up with int4 weights sharing one packed activation
    (convrot_linear_w4_gated); ``workspace`` as in ``linear_w4``."""
    dev = act_in.q.device
    out = _out_and_bias(act_in.rows, w_gate.rows, dev, out, out_dtype, b_gate)
    _check_bias(b_up, w_up.rows, dev, "b_up")
    ws = _w4_workspace(W4_GATED, act_in.rows, w_gate.rows, w_gate.K, dev, workspace)
    a, g, u = act_in.descriptor(), w_gate.descriptor(), w_up.descriptor()
    wp, wn = _ws(ws, dev)
    lib = _lib.load()
    _lib.check(lib.convrot_linear_w4_gated(
        ctypes.byref(a), ctypes.byref(g), _ptr(b_gate), ctypes.byref(u), _ptr(b_up), _act_code(act),
        out.data_ptr(), _DT[out.dtype], _ld(out), wp, wn, _stream(dev)))
    return out


def unpack_w4(w: PackedW4, out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 codes [rows, K] of an int4 weight (convrot_unpack_w4)."""
    if out is None:
        out = torch.empty((w.rows, w.K), dtype=torch.int8, device=w.q.device)
    desc = w.descriptor()
    lib = _lib.load()
    _lib.check(lib.convrot_unpack_w4(ctypes.byref(desc), out.data_ptr(), _ld(out), _stream(out.device)))
    return out


# ---------------------------------------------------------------------------
# Data-free smoothing of an FFN's intermediate channels (offline)
# ---------------------------------------------------------------------------

_SMOOTH = {"l2": _lib.SMOOTH_L2, "max": _lib.SMOOTH_MAX}



def tile_weight(w: Packed) -> Packed:
    """A copy of a packed weight in the TILE16 layout (convrot_tile_weight):
    16-row tiles whose 64-byte K units are each 1 KiB of consecutive memory,
    which the small-M path (M <= 16) streams faster.  Only M <= 16 calls
    accept it; keep the ROWS weight for larger M.  Needs N % 16 == 0 and
    K % 64 == 0."""
    if w.layout != ROWS:
        raise ValueError("tile_weight takes a ROWS weight")
    dev = w.q.device
    out = Packed(torch.empty((w.rows, w.K), dtype=torch.int8, device=dev), torch.empty_like(w.scale), w.group, w.kind,
                 w.signs, TILE16)
    lib = _lib.load()
    _lib.check(lib.convrot_tile_weight(ctypes.byref(w.descriptor()), ctypes.byref(out.descriptor()), _stream(dev)))
    return out


def tile_weight_w4(w: PackedW4) -> PackedW4:
    """tile_weight for int4 weights (convrot_tile_weight_w4; K % 128 == 0)."""
    if w.layout != ROWS:
        raise ValueError("tile_weight_w4 takes a ROWS weight")
    dev = w.q.device
    out = PackedW4(torch.empty((w.rows, w.K // 2), dtype=torch.uint8, device=dev), torch.empty_like(w.scale), w.K,
                   w.group, w.kind, w.signs, TILE16)
    lib = _lib.load()
    _lib.check(lib.convrot_tile_weight_w4(ctypes.byref(w.descriptor()), ctypes.byref(out.descriptor()),
                                          _stream(dev)))
    return out

def smooth_ffn(w_up: torch.Tensor, w_down: torch.Tensor, norm: str = "l2", scaled: bool = True):
    """s [F] = sqrt(n_up / n_down) per intermediate channel and, with
    ``scaled``, the fp32 weights W_up / s (rows) and W_down * s (columns)
    ready to pack (convrot_smooth_ffn).  Returns (s, up, down) or s."""
    for t, name in ((w_up, "w_up"), (w_down, "w_down")):
        _need_cuda(t, name)
        if t.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"{name} must be float32 or bfloat16")
    if norm not in _SMOOTH:
        raise ValueError(f"norm must be one of {sorted(_SMOOTH)}")
    F, K = w_up.shape
    K_out = w_down.shape[0]
    if w_down.shape[1] != F:
        raise ValueError("w_down must be [K_out, F] with F = w_up.shape[0]")
    dev = w_up.device
    s = torch.empty(F, dtype=torch.float32, device=dev)
    up = torch.empty((F, K), dtype=torch.float32, device=dev) if scaled else None
    dn = torch.empty((K_out, F), dtype=torch.float32, device=dev) if scaled else None
    lib = _lib.load()
    _lib.check(lib.convrot_smooth_ffn(
        w_up.data_ptr(), _DT[w_up.dtype], _ld(w_up), w_down.data_ptr(), _DT[w_down.dtype], _ld(w_down), F, K, K_out,
        _SMOOTH[norm], s.data_ptr(), up.data_ptr() if up is not None else None, _ld(up) if up is not None else 0,
        dn.data_ptr() if dn is not None else None, _ld(dn) if dn is not None else 0, _stream(dev)))
    return (s, up, dn) if scaled else s


# ---------------------------------------------------------------------------
# Runtime LoRA correction
# ---------------------------------------------------------------------------

def lora_workspace_bytes(M: int, K: int, r: int) -> int:
    """Bytes of device workspace ``lora_add`` needs for an input [M, K] and
    rank r on the current device (convrot_lora_workspace_bytes)."""
    lib = _lib.load()
    out = ctypes.c_int64(0)
    _lib.check(lib.convrot_lora_workspace_bytes(M, K, r, ctypes.byref(out)))
    return out.value


def lora_add(x: torch.Tensor, a: torch.Tensor, b: torch.Tensor, scale: float, y: torch.Tensor,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y += scale * (x a^T) b^T in place, from the unrotated bf16 input x
    [M, K], the adapter's down a [r, K] and up b [N, r] (convrot_lora_add).
    The rank-r intermediate T (bf16 [M, r]) is left at the start of
    ``workspace``, which holds at least ``lora_workspace_bytes(M, K, r)``
    bytes (allocated here when not given)."""
    for t, name in ((x, "x"), (a, "a"), (b, "b")):
        _need_cuda(t, name)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    M, K = x.shape
    r = a.shape[0]
    N = b.shape[0]
    if a.shape[1] != K or b.shape[1] != r or tuple(y.shape) != (M, N):
        raise ValueError("shapes must be x [M, K], a [r, K], b [N, r], y [M, N]")
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("y must be float32 or bfloat16")
    if workspace is None:
        with torch.cuda.device(x.device):
            workspace = torch.empty((max(lora_workspace_bytes(M, K, r), 16),), dtype=torch.uint8, device=x.device)
    lib = _lib.load()
    _lib.check(lib.convrot_lora_add(x.data_ptr(), _ld(x), M, K, a.data_ptr(), _ld(a), b.data_ptr(), _ld(b), N, r,
                                    float(scale), y.data_ptr(), _DT[y.dtype], _ld(y), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(x.device)))
    return y
