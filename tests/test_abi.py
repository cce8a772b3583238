"""The C ABI library on the host: it loads, exports every entry point that
include/convrot.h declares, and rejects bad arguments before launching
anything (CPU only: no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from w8a8_int8_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")

# Fake, 16-byte aligned "device" addresses: validation never dereferences them.
A16 = 0x10000
A16B = 0x20000
A16C = 0x30000
MIS = 0x10008


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(convrot_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_header():
    """libconvrot_probe.so (bench.py's hardware probes) exports exactly what
    include/convrot_probe.h declares, and rejects bad arguments on the host."""
    from w8a8_int8_linear_amd import probe

    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "convrot_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(convrot_[a-z0-9_]+)\s*\(", src)))
    assert names == sorted(probe.EXPORTED)
    plib = probe.load()
    f = plib.convrot_probe_mfma_i8
    assert f(None, 256, 10, A16, A16B, 0, None) == 1
    assert f(A16, 0, 10, A16, A16B, 0, None) == 1
    assert f(MIS, 256, 10, A16, A16B, 0, None) == 1
    r = plib.convrot_probe_read
    assert r(None, 1024, 8, A16, 0, None) == 1
    assert r(A16, 1000, 8, A16, 0, None) == 1
    assert r(MIS, 1024, 8, A16, 0, None) == 1
    assert r(A16, 1024, 0, A16, 0, None) == 1
    c = plib.convrot_probe_copy
    assert c(A16, A16, 1000, 8, None) == 1
    assert c(MIS, A16, 1024, 8, None) == 1


def test_abi_version_matches_header(lib):
    src = open(HEADER).read()
    v = int(re.search(r"#define CONVROT_ABI_VERSION (\d+)", src).group(1))
    assert lib.convrot_abi_version() == v == _lib.ABI_VERSION


def test_status_strings(lib):
    for code, name in enumerate(["CONVROT_OK", "CONVROT_ERR_INVALID_ARG", "CONVROT_ERR_GROUP", "CONVROT_ERR_DTYPE",
                                 "CONVROT_ERR_ALIGN", "CONVROT_ERR_MISMATCH", "CONVROT_ERR_HIP"]):
        assert lib.convrot_status_string(code).decode() == name


def test_struct_layout():
    assert ctypes.sizeof(_lib.Rot) == 16
    assert ctypes.sizeof(_lib.Packed) == 64
    assert _lib.Packed.rot.offset == 40
    assert _lib.Packed.layout.offset == 56


def packed(rows=4, K=256, ld=None, G=256, kind=_lib.ROT_REGULAR, signs=None, q=A16, scale=A16B,
           layout=_lib.LAYOUT_ROWS):
    return _lib.Packed(q, scale, rows, K, ld if ld is not None else K, _lib.Rot(G, kind, signs), layout)


def pack_status(lib, X=A16C, xdt=_lib.BF16, ldx=None, out=None):
    out = out if out is not None else packed()
    return lib.convrot_pack_act(X, xdt, ldx if ldx is not None else out.K, ctypes.byref(out), None)


@pytest.mark.parametrize("G", [2, 8, 32, 128, 512, 2048, 0, -4])
def test_pack_rejects_regular_group(lib, G):
    assert pack_status(lib, out=packed(K=4096, G=G)) == _lib.ERR_GROUP


def test_pack_rejects_k_not_multiple_of_g(lib):
    assert pack_status(lib, out=packed(K=2688, G=256)) == _lib.ERR_GROUP
    assert b"2688" in lib.convrot_last_error()


def test_pack_rejects_k_not_multiple_of_16(lib):
    assert pack_status(lib, out=packed(K=1028, G=4)) == _lib.ERR_INVALID_ARG


def test_pack_rejects_k_too_large(lib):
    assert pack_status(lib, out=packed(K=65536 + 1024, G=1024)) == _lib.ERR_INVALID_ARG


def test_pack_rejects_dtype(lib):
    assert pack_status(lib, xdt=_lib.I32) == _lib.ERR_DTYPE
    assert pack_status(lib, xdt=7) == _lib.ERR_DTYPE


def test_pack_rejects_null_and_misaligned(lib):
    assert pack_status(lib, X=None) == _lib.ERR_INVALID_ARG
    assert pack_status(lib, out=packed(q=None)) == _lib.ERR_INVALID_ARG
    assert pack_status(lib, out=packed(scale=None)) == _lib.ERR_INVALID_ARG
    assert pack_status(lib, X=MIS) == _lib.ERR_ALIGN
    assert pack_status(lib, out=packed(q=MIS)) == _lib.ERR_ALIGN
    assert pack_status(lib, out=packed(scale=A16B + 2)) == _lib.ERR_ALIGN
    assert lib.convrot_pack_act(A16C, _lib.BF16, 256, None, None) == _lib.ERR_INVALID_ARG


def test_pack_rejects_bad_leading_dimensions(lib):
    assert pack_status(lib, ldx=128) == _lib.ERR_INVALID_ARG        # ld < K
    assert pack_status(lib, ldx=260) == _lib.ERR_ALIGN               # 520 bytes
    assert pack_status(lib, out=packed(ld=264)) == _lib.ERR_ALIGN    # int8 ld % 16
    assert pack_status(lib, out=packed(ld=200)) == _lib.ERR_INVALID_ARG


def test_pack_rotation_kind_and_signs(lib):
    assert pack_status(lib, out=packed(G=128, kind=_lib.ROT_RANDOMIZED, K=1152)) == _lib.ERR_INVALID_ARG
    assert pack_status(lib, out=packed(G=256, signs=A16)) == _lib.ERR_INVALID_ARG
    assert pack_status(lib, out=packed(G=128, kind=_lib.ROT_RANDOMIZED, K=1152, signs=MIS)) == _lib.ERR_ALIGN
    assert pack_status(lib, out=packed(G=8, kind=_lib.ROT_RANDOMIZED, K=1152, signs=A16)) == _lib.ERR_GROUP
    assert pack_status(lib, out=packed(G=2048, kind=_lib.ROT_RANDOMIZED, K=4096, signs=A16)) == _lib.ERR_GROUP
    assert pack_status(lib, out=packed(kind=5)) == _lib.ERR_INVALID_ARG


def test_pack_zero_rows_is_a_no_op(lib):
    assert pack_status(lib, out=packed(rows=0)) == _lib.OK
    assert lib.convrot_last_error() == b""
    assert pack_status(lib, out=packed(rows=-1)) == _lib.ERR_INVALID_ARG


def linear_status(lib, act=None, w=None, bias=None, Y=A16C, ydt=_lib.BF16, ldy=None, ws=None, ws_bytes=0):
    act = act if act is not None else packed(rows=32)
    w = w if w is not None else packed(rows=64, q=0x40000, scale=0x50000)
    return lib.convrot_linear(ctypes.byref(act), ctypes.byref(w), bias, Y, ydt,
                              ldy if ldy is not None else w.rows, ws, ws_bytes, None)


def test_linear_mismatch(lib):
    assert linear_status(lib, w=packed(rows=64, K=512, q=0x40000)) == _lib.ERR_MISMATCH
    assert linear_status(lib, w=packed(rows=64, G=64, q=0x40000)) == _lib.ERR_MISMATCH
    a = packed(rows=32, G=128, kind=_lib.ROT_RANDOMIZED, K=1152, signs=0x60000)
    w = packed(rows=64, G=128, kind=_lib.ROT_RANDOMIZED, K=1152, signs=0x70000, q=0x40000)
    assert linear_status(lib, act=a, w=w) == _lib.ERR_MISMATCH
    a2 = packed(rows=32, G=16, K=1152)
    assert linear_status(lib, act=a2, w=packed(rows=64, G=16, kind=_lib.ROT_RANDOMIZED, K=1152,
                                                 signs=0x60000, q=0x40000)) == _lib.ERR_MISMATCH


def test_linear_output_checks(lib):
    assert linear_status(lib, ydt=9) == _lib.ERR_DTYPE
    assert linear_status(lib, Y=None) == _lib.ERR_INVALID_ARG
    assert linear_status(lib, Y=A16C + 1) == _lib.ERR_ALIGN        # not element aligned
    assert linear_status(lib, Y=A16C + 2, ydt=_lib.F32) == _lib.ERR_ALIGN
    assert linear_status(lib, ldy=32) == _lib.ERR_INVALID_ARG     # ldy < N
    assert linear_status(lib, bias=A16 + 2) == _lib.ERR_ALIGN
    assert lib.convrot_linear(None, None, None, A16C, _lib.BF16, 64, None, 0, None) == _lib.ERR_INVALID_ARG


def test_linear_empty_is_a_no_op(lib):
    assert linear_status(lib, act=packed(rows=0)) == _lib.OK
    assert linear_status(lib, w=packed(rows=0, q=0x40000), ldy=0) == _lib.OK


def test_linear_k_overflow_guard(lib):
    K = 1024 * 1024
    assert linear_status(lib, act=packed(rows=4, K=K, G=1024),
                         w=packed(rows=4, K=K, G=1024, q=0x40000)) == _lib.ERR_INVALID_ARG


def act_status(lib, fn=_lib.ACT_GELU_ERF, ydt=_lib.BF16, act=None, w=None):
    act = act if act is not None else packed(rows=32)
    w = w if w is not None else packed(rows=64, q=0x40000, scale=0x50000)
    return lib.convrot_linear_act(ctypes.byref(act), ctypes.byref(w), None, fn, A16C, ydt, w.rows, None, 0, None)


def gated_status(lib, fn=_lib.ACT_GELU_TANH, ydt=_lib.BF16, up=None, gate=None):
    act = packed(rows=8)
    g = gate if gate is not None else packed(rows=64, q=0x40000, scale=0x50000)
    u = up if up is not None else packed(rows=64, q=0x80000, scale=0x90000)
    return lib.convrot_linear_gated(ctypes.byref(act), ctypes.byref(g), None, ctypes.byref(u), None, fn, A16C, ydt,
                                    g.rows, None, 0, None)


def test_linear_act_checks(lib):
    assert act_status(lib, fn=_lib.ACT_NONE) == _lib.ERR_INVALID_ARG
    assert act_status(lib, fn=7) == _lib.ERR_INVALID_ARG
    assert act_status(lib, ydt=_lib.I32) == _lib.ERR_DTYPE        # an activation needs a float output
    assert act_status(lib, w=packed(rows=64, K=512, q=0x40000)) == _lib.ERR_MISMATCH
    assert act_status(lib, act=packed(rows=0)) == _lib.OK


def test_linear_gated_checks(lib):
    assert gated_status(lib, fn=_lib.ACT_NONE) == _lib.ERR_INVALID_ARG
    assert gated_status(lib, ydt=_lib.I32) == _lib.ERR_DTYPE
    assert gated_status(lib, up=packed(rows=63, q=0x80000)) == _lib.ERR_MISMATCH      # N differs
    assert gated_status(lib, up=packed(rows=64, G=64, q=0x80000)) == _lib.ERR_MISMATCH  # rotation differs
    assert gated_status(lib, gate=packed(rows=64, K=512, q=0x40000)) == _lib.ERR_MISMATCH
    assert lib.convrot_linear_gated(None, None, None, None, None, _lib.ACT_GELU_TANH, A16C, _lib.BF16, 64,
                                    None, 0, None) == _lib.ERR_INVALID_ARG


def test_linear_bf16_checks(lib):
    def f(*a):
        return lib.convrot_linear_bf16(*a, None, 0, None)
    assert f(A16, 2688, A16B, 2688, None, 8, 16, 2690, A16C, _lib.BF16, 16) == _lib.ERR_INVALID_ARG
    assert f(A16, 2688, A16B, 2688, None, 8, 16, 2688, A16C, _lib.I32, 16) == _lib.ERR_DTYPE
    assert f(None, 2688, A16B, 2688, None, 8, 16, 2688, A16C, _lib.BF16, 16) == _lib.ERR_INVALID_ARG
    assert f(A16, 2684, A16B, 2688, None, 8, 16, 2688, A16C, _lib.BF16, 16) == _lib.ERR_INVALID_ARG
    assert f(A16, 2688, A16B, 2688, None, 0, 16, 2688, A16C, _lib.BF16, 16) == _lib.OK


def ws_bytes(lib, kind, M, N, K):
    out = ctypes.c_int64(-1)
    st = lib.convrot_linear_workspace_bytes(kind, M, N, K, ctypes.byref(out))
    return st, out.value


def test_linear_workspace_query(lib):
    """Small M: the split-K partials (the down projection's 72 tiles split,
    the gated pair's 432 tiles do not); large M: nothing, except the int4
    kinds' expanded weight.  The device's CU count enters the size (no GPU
    here: the library assumes 256)."""
    st, down = ws_bytes(lib, _lib.LINEAR_PLAIN, 16, 1152, 6912)
    assert st == _lib.OK and down > 0 and down % 1024 == 0
    assert ws_bytes(lib, _lib.LINEAR_GATED, 16, 6912, 1152) == (_lib.OK, 0)
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 17, 1152, 6912) == (_lib.OK, 0)
    assert ws_bytes(lib, _lib.LINEAR_W4, 17, 1152, 6912) == (_lib.OK, 1152 * 6912)
    assert ws_bytes(lib, _lib.LINEAR_W4, 16, 1152, 6912) == (_lib.OK, 0)      # int4 small M never splits
    assert ws_bytes(lib, _lib.LINEAR_W4_GATED, 64, 6912, 1152) == (_lib.OK, 2 * 6912 * 1152)
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 0, 1152, 6912) == (_lib.OK, 0)
    assert ws_bytes(lib, _lib.LINEAR_GATED, 16, 1152, 6912)[1] == 2 * down   # two weights' partials
    assert ws_bytes(lib, _lib.LINEAR_BF16, 16, 1152, 6912)[1] > 0
    # up to 12 rows, a plain int8 launch with fewer tiles than CUs and at
    # least 32 K units takes one 16-wave workgroup per tile and no split
    for m in (1, 4, 12):
        assert ws_bytes(lib, _lib.LINEAR_PLAIN, m, 1152, 6912) == (_lib.OK, 0)
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 13, 1152, 6912) == (_lib.OK, down)
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 4, 1152, 1984)[1] > 0          # 31 K units: split
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 4, 1152, 2048) == (_lib.OK, 0)
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 4, 4096, 6912) == (_lib.OK, 0)  # 256 tiles: no split either way
    assert ws_bytes(lib, _lib.LINEAR_GATED, 1, 1152, 6912)[1] == 2 * down   # gated and bf16 keep the split
    assert ws_bytes(lib, _lib.LINEAR_BF16, 1, 1152, 6912)[1] > 0
    assert ws_bytes(lib, 9, 16, 1152, 6912)[0] == _lib.ERR_INVALID_ARG
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, 16, 1152, 6913)[0] == _lib.ERR_INVALID_ARG
    assert ws_bytes(lib, _lib.LINEAR_PLAIN, -1, 1152, 6912)[0] == _lib.ERR_INVALID_ARG
    assert lib.convrot_linear_workspace_bytes(_lib.LINEAR_PLAIN, 16, 1152, 6912, None) == _lib.ERR_INVALID_ARG


def test_linear_noalloc_checks(lib):
    """The no-allocation variant validates like convrot_linear before it
    touches its scratch."""
    f = lib.convrot_linear_noalloc
    act, w = packed(rows=16, K=6912), packed(rows=1152, K=6912, q=0x40000, scale=0x50000)
    assert f(None, None, None, A16C, _lib.BF16, 64, None) == _lib.ERR_INVALID_ARG
    assert f(ctypes.byref(act), ctypes.byref(packed(rows=1152, K=3072, q=0x40000)), None, A16C, _lib.BF16, 1152,
             None) == _lib.ERR_MISMATCH
    assert f(ctypes.byref(act), ctypes.byref(w), None, A16C, 9, 1152, None) == _lib.ERR_DTYPE
    assert f(ctypes.byref(act), ctypes.byref(w), None, A16C, _lib.BF16, 1000, None) == _lib.ERR_INVALID_ARG
    assert f(ctypes.byref(packed(rows=0, K=6912)), ctypes.byref(w), None, A16C, _lib.BF16, 1152, None) == _lib.OK
    # the largest split of this entry point fits its static scratch on a 256-CU GPU
    worst = max(ws_bytes(lib, _lib.LINEAR_PLAIN, 16, n, 12288)[1] for n in range(16, 4096, 16))
    assert 0 < worst <= _lib.NOALLOC_SCRATCH_BYTES


def test_rowmax_entry_point_checks(lib):
    """Producer-fusion entry points validate on the host before any launch."""
    f = lib.convrot_linear_act_rowmax

    def st(group=256, N=512, M=64, Y=A16C, ldy=512, ldm=2, rowmax=0x60000, fn=_lib.ACT_GELU_ERF):
        a = packed(rows=M, K=1024)
        ww = packed(rows=N, K=1024, q=0x40000, scale=0x50000)
        return f(ctypes.byref(a), ctypes.byref(ww), None, fn, Y, _lib.BF16, ldy, group, rowmax, ldm, None)
    assert st(group=128) == _lib.ERR_GROUP
    assert st(group=1024, ldm=1) == _lib.ERR_GROUP
    assert st(N=320, ldy=320) == _lib.ERR_INVALID_ARG      # N % 256
    assert st(M=16) == _lib.ERR_INVALID_ARG                 # small M
    assert st(ldm=1) == _lib.ERR_INVALID_ARG                # ldm < N / G
    assert st(Y=A16C + 2) == _lib.ERR_ALIGN                 # rows not aligned for 4-element stores
    assert st(rowmax=None) == _lib.ERR_INVALID_ARG
    assert st(fn=_lib.ACT_NONE) == _lib.ERR_INVALID_ARG
    assert st(M=0) == _lib.OK
    g = lib.convrot_pack_act_rowmax
    out = packed(rows=8, K=1024, G=256)
    assert g(A16C, _lib.BF16, 1024, 0x60000, 3, ctypes.byref(out), None) == _lib.ERR_INVALID_ARG   # ldm < K / G
    big = packed(rows=8, K=2048, G=1024)
    assert g(A16C, _lib.BF16, 2048, 0x60000, 2, ctypes.byref(big), None) == _lib.ERR_GROUP
    rnd = packed(rows=8, K=1024, G=256, kind=_lib.ROT_RANDOMIZED, signs=0x70000)
    assert g(A16C, _lib.BF16, 1024, 0x60000, 4, ctypes.byref(rnd), None) == _lib.ERR_GROUP
    assert g(A16C, _lib.BF16, 1024, 0x60000, 4, ctypes.byref(packed(rows=0, K=1024)), None) == _lib.OK


def test_linear_rejects_a_short_workspace(lib):
    """A non-NULL workspace smaller than the split needs is an error before
    any launch (NULL would select the unsplit kernel)."""
    K, N = 6912, 1152
    need = ws_bytes(lib, _lib.LINEAR_PLAIN, 16, N, K)[1]
    act = packed(rows=16, K=K)
    w = packed(rows=N, K=K, q=0x40000, scale=0x50000)
    assert linear_status(lib, act=act, w=w, ws=0x100000, ws_bytes=need - 1) == _lib.ERR_INVALID_ARG
    assert b"workspace" in lib.convrot_last_error()
    assert linear_status(lib, act=act, w=w, ws=0x100008, ws_bytes=need) == _lib.ERR_ALIGN
    f = lib.convrot_linear_act
    assert f(ctypes.byref(act), ctypes.byref(w), None, _lib.ACT_GELU_ERF, A16C, _lib.BF16, N, 0x100000, need - 1,
             None) == _lib.ERR_INVALID_ARG
    assert lib.convrot_linear_bf16(A16, K, A16B, K, None, 16, N, K, A16C, _lib.BF16, N, 0x100000, 16,
                                   None) == _lib.ERR_INVALID_ARG



def test_rotate_checks(lib):
    f = lib.convrot_rotate
    rot = _lib.Rot(256, _lib.ROT_REGULAR, None)
    assert f(A16, _lib.BF16, 4, 2688, 2688, rot, A16B, 2688, None) == _lib.ERR_GROUP
    assert f(A16, _lib.BF16, 4, 1024, 1024, rot, MIS, 1024, None) == _lib.ERR_ALIGN
    assert f(A16, _lib.BF16, 0, 1024, 1024, rot, A16B, 1024, None) == _lib.OK


def test_error_string_is_cleared_by_success(lib):
    assert pack_status(lib, out=packed(K=2688)) == _lib.ERR_GROUP
    assert lib.convrot_last_error() != b""
    assert pack_status(lib, out=packed(rows=0)) == _lib.OK
    assert lib.convrot_last_error() == b""


def test_python_layer_raises_on_error():
    with pytest.raises(_lib.ConvrotError) as e:
        _lib.check(_lib.ERR_GROUP)
    assert e.value.status == _lib.ERR_GROUP


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "nope.so"))


# -- int4 weights (W4A8) -------------------------------------------------------

def packed_w4(rows=64, K=256, ld=None, G=256, kind=_lib.ROT_REGULAR, signs=None, q=0x40000, scale=0x50000,
              layout=_lib.LAYOUT_ROWS):
    return _lib.PackedW4(q, scale, rows, K, ld if ld is not None else K // 2, _lib.Rot(G, kind, signs), layout)


def test_w4_struct_layout():
    assert ctypes.sizeof(_lib.PackedW4) == ctypes.sizeof(_lib.Packed) == 64
    assert _lib.PackedW4.rot.offset == 40
    assert _lib.PackedW4.layout.offset == 56


def w4_status(lib, act=None, w=None, fn=_lib.ACT_NONE, ydt=_lib.BF16, ws=None, ws_bytes=0):
    act = act if act is not None else packed(rows=32)
    w = w if w is not None else packed_w4()
    return lib.convrot_linear_w4(ctypes.byref(act), ctypes.byref(w), None, fn, A16C, ydt, w.rows, ws, ws_bytes, None)


def test_w4_pack_checks(lib):
    def st(out, wdt=_lib.BF16, ldw=256):
        return lib.convrot_pack_weight_w4(A16C, wdt, ldw, ctypes.byref(out), None)
    assert st(packed_w4(ld=120)) == _lib.ERR_INVALID_ARG      # ld < K / 2
    assert st(packed_w4(ld=132)) == _lib.ERR_ALIGN            # ld % 8
    # an 8-byte pitch passes the descriptor checks (the dtype check after them fails)
    assert st(packed_w4(ld=136), wdt=_lib.I32) == _lib.ERR_DTYPE
    assert st(packed_w4(q=MIS)) == _lib.ERR_ALIGN
    assert st(packed_w4(G=128)) == _lib.ERR_GROUP
    assert st(packed_w4(), wdt=_lib.I32) == _lib.ERR_DTYPE
    assert st(packed_w4(rows=0)) == _lib.OK


def test_w4_linear_needs_a_workspace_above_16_rows(lib):
    assert w4_status(lib) == _lib.ERR_INVALID_ARG
    assert b"workspace" in lib.convrot_last_error()
    assert w4_status(lib, ws=0x80000, ws_bytes=64 * 256 - 1) == _lib.ERR_INVALID_ARG
    assert w4_status(lib, ws=0x80008, ws_bytes=64 * 256) == _lib.ERR_ALIGN


def test_w4_linear_checks(lib):
    assert w4_status(lib, w=packed_w4(K=512, ld=256)) == _lib.ERR_MISMATCH
    assert w4_status(lib, w=packed_w4(G=64)) == _lib.ERR_MISMATCH
    assert w4_status(lib, fn=7) == _lib.ERR_INVALID_ARG
    assert w4_status(lib, fn=_lib.ACT_GELU_ERF, ydt=_lib.I32) == _lib.ERR_DTYPE
    assert w4_status(lib, act=packed(rows=0)) == _lib.OK
    g = packed_w4()
    u = packed_w4(rows=32, q=0x90000, scale=0xA0000)
    act = packed(rows=8)
    assert lib.convrot_linear_w4_gated(ctypes.byref(act), ctypes.byref(g), None, ctypes.byref(u), None,
                                       _lib.ACT_GELU_TANH, A16C, _lib.BF16, 64, None, 0, None) == _lib.ERR_MISMATCH
    assert lib.convrot_linear_w4_gated(ctypes.byref(act), ctypes.byref(g), None, ctypes.byref(g), None,
                                       _lib.ACT_NONE, A16C, _lib.BF16, 64, None, 0, None) == _lib.ERR_INVALID_ARG


def test_w4_unpack_checks(lib):
    w = packed_w4()
    assert lib.convrot_unpack_w4(ctypes.byref(w), A16C, 128, None) == _lib.ERR_INVALID_ARG  # ldd < K
    assert lib.convrot_unpack_w4(ctypes.byref(w), MIS, 256, None) == _lib.ERR_ALIGN
    assert lib.convrot_unpack_w4(ctypes.byref(packed_w4(rows=0)), A16C, 256, None) == _lib.OK



# -- data-free smoothing ------------------------------------------------------

def smooth_status(lib, up=A16, up_dt=_lib.BF16, ldu=64, dn=A16B, dn_dt=_lib.BF16, ldd=32, F=32, K=64, K_out=48,
                  norm=_lib.SMOOTH_L2, s=A16C, uo=None, lduo=0, do=None, lddo=0):
    return lib.convrot_smooth_ffn(up, up_dt, ldu, dn, dn_dt, ldd, F, K, K_out, norm, s, uo, lduo, do, lddo, None)


def test_smooth_checks(lib):
    assert smooth_status(lib, F=0) == _lib.OK
    assert smooth_status(lib, up_dt=_lib.I32) == _lib.ERR_DTYPE
    assert smooth_status(lib, norm=3) == _lib.ERR_INVALID_ARG
    assert smooth_status(lib, s=None) == _lib.ERR_INVALID_ARG
    assert smooth_status(lib, s=A16C + 2) == _lib.ERR_ALIGN
    assert smooth_status(lib, ldu=32) == _lib.ERR_INVALID_ARG          # ldu < K
    assert smooth_status(lib, ldd=16) == _lib.ERR_INVALID_ARG          # ldd < F
    assert smooth_status(lib, up=A16 + 1) == _lib.ERR_ALIGN            # bf16 element alignment
    assert smooth_status(lib, uo=0x40000, lduo=32) == _lib.ERR_INVALID_ARG
    assert smooth_status(lib, do=0x50000, lddo=16) == _lib.ERR_INVALID_ARG
    assert smooth_status(lib, F=-1) == _lib.ERR_INVALID_ARG



# -- runtime LoRA correction ----------------------------------------------------

def lora_status(lib, X=A16, ldx=64, M=32, K=64, A=A16B, lda=64, B=A16C, ldb=16, N=48, r=16, Y=0x40000,
                ydt=_lib.BF16, ldy=48, ws=0x50000, ws_bytes=32 * 16 * 2):
    return lib.convrot_lora_add(X, ldx, M, K, A, lda, B, ldb, N, r, ctypes.c_float(0.5), Y, ydt, ldy, ws, ws_bytes,
                                None)


def test_lora_checks(lib):
    assert lora_status(lib, r=8) == _lib.ERR_INVALID_ARG
    assert lora_status(lib, r=0) == _lib.ERR_INVALID_ARG
    assert lora_status(lib, r=272, ldb=272) == _lib.ERR_INVALID_ARG   # rank above 256
    assert lora_status(lib, K=40, ldx=40, lda=40) == _lib.ERR_INVALID_ARG
    assert lora_status(lib, ydt=_lib.I32) == _lib.ERR_DTYPE
    assert lora_status(lib, X=MIS) == _lib.ERR_ALIGN
    assert lora_status(lib, ldb=12) == _lib.ERR_INVALID_ARG           # ldb < r
    assert lora_status(lib, ldb=20) == _lib.ERR_ALIGN                 # 40-byte rows
    assert lora_status(lib, ws=None) == _lib.ERR_INVALID_ARG
    assert lora_status(lib, ws_bytes=32 * 16 * 2 - 2) == _lib.ERR_INVALID_ARG
    assert lora_status(lib, ws=0x50008) == _lib.ERR_ALIGN
    assert lora_status(lib, M=0) == _lib.OK


def lora_ws(lib, M, K, r):
    out = ctypes.c_int64(-1)
    st = lib.convrot_lora_workspace_bytes(M, K, r, ctypes.byref(out))
    return st, out.value


def test_lora_workspace_query(lib):
    # one K block: bf16 T only, rounded up to 256 bytes
    assert lora_ws(lib, 32, 64, 16) == (_lib.OK, 1024)
    assert lora_ws(lib, 3, 64, 16) == (_lib.OK, 256)
    assert lora_ws(lib, 0, 64, 16) == (_lib.OK, 0)
    # 4096 rows of K = 3072 at r = 32 split K into 4 blocks on 256 CUs:
    # T (256 KiB) plus 4 x 4096 x 32 fp32 partials
    st, n = lora_ws(lib, 4096, 3072, 32)
    assert st == _lib.OK and n >= 4096 * 32 * 2 and (n - 4096 * 32 * 2) % (4096 * 32 * 4) == 0
    assert lora_ws(lib, 32, 64, 8)[0] == _lib.ERR_INVALID_ARG
    assert lora_ws(lib, 32, 40, 16)[0] == _lib.ERR_INVALID_ARG
    assert lora_ws(lib, -1, 64, 16)[0] == _lib.ERR_INVALID_ARG
    assert lib.convrot_lora_workspace_bytes(32, 64, 16, None) == _lib.ERR_INVALID_ARG
    # the call itself rejects a workspace one byte short of the query
    assert lora_status(lib, M=4096, ldx=3072, K=3072, lda=3072, r=32, ldb=32, N=48, ldy=48, ws_bytes=n - 1) \
        == _lib.ERR_INVALID_ARG


# -- TILE16 weight layout -------------------------------------------------------
# Every case below is rejected on the host before any launch.

T16 = _lib.LAYOUT_TILE16


def tile_status(lib, src=None, dst=None):
    src = src if src is not None else packed(rows=64, q=0x40000, scale=0x50000)
    dst = dst if dst is not None else packed(rows=64, q=0x80000, scale=0x90000, layout=T16)
    return lib.convrot_tile_weight(ctypes.byref(src), ctypes.byref(dst), None)


def test_tile_weight_checks(lib):
    assert lib.convrot_tile_weight(None, None, None) == _lib.ERR_INVALID_ARG
    assert tile_status(lib, dst=packed(rows=64, q=0x80000, scale=0x90000)) == _lib.ERR_INVALID_ARG  # ROWS output
    assert b"TILE16" in lib.convrot_last_error()
    assert tile_status(lib, src=packed(rows=64, q=0x40000, layout=T16)) == _lib.ERR_INVALID_ARG     # tiled input
    assert tile_status(lib, dst=packed(rows=60, q=0x80000, layout=T16)) == _lib.ERR_INVALID_ARG     # rows % 16
    assert tile_status(lib, dst=packed(rows=64, ld=512, q=0x80000, layout=T16)) == _lib.ERR_INVALID_ARG  # padded
    assert tile_status(lib, src=packed(rows=64, K=96, G=16, q=0x40000),
                       dst=packed(rows=64, K=96, G=16, q=0x80000, layout=T16)) == _lib.ERR_INVALID_ARG  # K % 64
    assert tile_status(lib, dst=packed(rows=64, q=0x80000, layout=2)) == _lib.ERR_INVALID_ARG       # unknown layout
    assert b"unknown layout" in lib.convrot_last_error()
    assert tile_status(lib, src=packed(rows=48, q=0x40000)) == _lib.ERR_MISMATCH
    assert tile_status(lib, src=packed(rows=64, K=512, q=0x40000),
                       dst=packed(rows=64, K=512, q=0x80000, layout=T16, G=64)) == _lib.ERR_MISMATCH
    # the tiled copy cannot be written over its own source
    assert tile_status(lib, dst=packed(rows=64, q=0x40000 + 64 * 256 - 16, layout=T16)) == _lib.ERR_INVALID_ARG
    assert b"overlap" in lib.convrot_last_error()
    assert tile_status(lib, src=packed(rows=0, q=0x40000), dst=packed(rows=0, q=0x80000, layout=T16)) == _lib.OK


def test_tile_weight_w4_checks(lib):
    def st(src=None, dst=None):
        src = src if src is not None else packed_w4()
        dst = dst if dst is not None else packed_w4(q=0x80000, scale=0x90000, layout=T16)
        return lib.convrot_tile_weight_w4(ctypes.byref(src), ctypes.byref(dst), None)
    assert st(dst=packed_w4(q=0x80000, scale=0x90000)) == _lib.ERR_INVALID_ARG
    assert st(dst=packed_w4(rows=56, q=0x80000, layout=T16)) == _lib.ERR_INVALID_ARG
    assert st(dst=packed_w4(ld=256, q=0x80000, layout=T16)) == _lib.ERR_INVALID_ARG
    assert st(src=packed_w4(rows=32)) == _lib.ERR_MISMATCH
    assert st(src=packed_w4(rows=0), dst=packed_w4(rows=0, q=0x80000, layout=T16)) == _lib.OK


def test_tiled_weight_serves_small_m_only(lib):
    tiled = packed(rows=64, q=0x40000, scale=0x50000, layout=T16)
    assert linear_status(lib, act=packed(rows=17), w=tiled) == _lib.ERR_INVALID_ARG
    assert b"M <= 16" in lib.convrot_last_error()
    assert act_status(lib, act=packed(rows=32), w=tiled) == _lib.ERR_INVALID_ARG
    assert w4_status(lib, w=packed_w4(layout=T16), ws=0x80000, ws_bytes=1 << 20) == _lib.ERR_INVALID_ARG
    assert b"M <= 16" in lib.convrot_last_error()
    # a tiled activation serves M <= 16 with int8 weights, dense rows and whole 64-byte units
    w = packed(rows=64, q=0x40000, scale=0x50000)
    assert linear_status(lib, act=packed(rows=17, layout=T16), w=w) == _lib.ERR_INVALID_ARG
    assert b"TILE16 activation serves M <= 16" in lib.convrot_last_error()
    assert linear_status(lib, act=packed(rows=16, ld=512, layout=T16), w=w) == _lib.ERR_INVALID_ARG
    assert b"ld == K" in lib.convrot_last_error()
    assert linear_status(lib, act=packed(rows=4, K=96, G=16, layout=T16),
                         w=packed(rows=64, K=96, G=16, q=0x40000, scale=0x50000)) == _lib.ERR_INVALID_ARG
    assert linear_status(lib, act=packed(rows=4, layout=3), w=w) == _lib.ERR_INVALID_ARG
    assert b"unknown layout" in lib.convrot_last_error()
    assert w4_status(lib, act=packed(rows=4, layout=T16), ws=0x80000, ws_bytes=1 << 20) == _lib.ERR_INVALID_ARG
    assert b"ROWS" in lib.convrot_last_error()


def test_gated_pairs_share_a_layout(lib):
    tiled = packed(rows=64, q=0x40000, scale=0x50000, layout=T16)
    assert gated_status(lib, gate=tiled) == _lib.ERR_INVALID_ARG
    assert b"same layout" in lib.convrot_last_error()
    g = packed_w4(layout=T16)
    u = packed_w4(q=0x90000, scale=0xA0000)
    act = packed(rows=8)
    assert lib.convrot_linear_w4_gated(ctypes.byref(act), ctypes.byref(g), None, ctypes.byref(u), None,
                                       _lib.ACT_GELU_TANH, A16C, _lib.BF16, 64, None, 0, None) == _lib.ERR_INVALID_ARG
    assert b"same layout" in lib.convrot_last_error()


def test_packing_and_unpacking_stay_in_rows(lib):
    # a packed activation may be tiled (dense rows, K % 64 == 0); a packed weight is written in rows
    assert pack_status(lib, out=packed(rows=16, ld=512, layout=T16)) == _lib.ERR_INVALID_ARG
    assert b"ld == K" in lib.convrot_last_error()
    assert pack_status(lib, out=packed(rows=4, K=96, G=16, layout=T16)) == _lib.ERR_INVALID_ARG
    assert lib.convrot_pack_weight(A16C, _lib.BF16, 256, ctypes.byref(packed(rows=16, layout=T16)),
                                   None) == _lib.ERR_INVALID_ARG
    assert b"ROWS" in lib.convrot_last_error()
    out = packed_w4(layout=T16)
    assert lib.convrot_pack_weight_w4(A16C, _lib.BF16, 256, ctypes.byref(out), None) == _lib.ERR_INVALID_ARG
    assert lib.convrot_unpack_w4(ctypes.byref(out), A16C, 256, None) == _lib.ERR_INVALID_ARG
    assert b"ROWS" in lib.convrot_last_error()


# -- linears that pack their own activation rows ----------------------------------

def packin_status(lib, X=A16C, xdt=_lib.BF16, ldx=256, M=1, w=None, fn=_lib.ACT_NONE, ydt=_lib.BF16, Y=0x90000,
                  ldy=None):
    w = w if w is not None else packed(rows=64, q=0x40000, scale=0x50000)
    return lib.convrot_linear_packin(X, xdt, ldx, M, ctypes.byref(w), None, fn, Y, ydt,
                                     ldy if ldy is not None else w.rows, None)


def gated_packin_status(lib, M=1, gate=None, up=None, fn=_lib.ACT_GELU_TANH, ydt=_lib.BF16, xdt=_lib.BF16, ldx=None):
    g = gate if gate is not None else packed(rows=64, q=0x40000, scale=0x50000)
    u = up if up is not None else packed(rows=64, q=0x80000, scale=0x90000)
    return lib.convrot_linear_gated_packin(A16C, xdt, ldx if ldx is not None else g.K, M, ctypes.byref(g), None,
                                           ctypes.byref(u), None, fn, 0xA0000, ydt, g.rows, None)


def test_packin_checks(lib):
    """Every rule is checked on the host before any launch."""
    assert packin_status(lib, M=5) == _lib.ERR_INVALID_ARG
    assert b"0 to 4 rows" in lib.convrot_last_error()
    assert packin_status(lib, M=-1) == _lib.ERR_INVALID_ARG
    assert packin_status(lib, xdt=_lib.F32) == _lib.ERR_DTYPE
    assert packin_status(lib, X=A16C + 8) == _lib.ERR_ALIGN            # rows read in 16-byte chunks
    assert packin_status(lib, ldx=252) == _lib.ERR_INVALID_ARG          # ldx < K
    assert packin_status(lib, ldx=260) == _lib.ERR_ALIGN                # 520-byte row pitch
    assert packin_status(lib, X=None) == _lib.ERR_INVALID_ARG
    assert packin_status(lib, fn=7) == _lib.ERR_INVALID_ARG
    assert packin_status(lib, fn=_lib.ACT_GELU_ERF, ydt=_lib.I32) == _lib.ERR_DTYPE
    assert packin_status(lib, ydt=9) == _lib.ERR_DTYPE
    assert packin_status(lib, Y=None) == _lib.ERR_INVALID_ARG
    assert packin_status(lib, ldy=32) == _lib.ERR_INVALID_ARG           # ldy < N
    big = packed(rows=64, K=16400, G=16, q=0x40000, scale=0x50000)
    assert packin_status(lib, w=big, ldx=16400) == _lib.ERR_INVALID_ARG
    assert b"16384" in lib.convrot_last_error()
    assert packin_status(lib, w=packed(rows=64, G=64, kind=9, q=0x40000)) == _lib.ERR_INVALID_ARG
    assert packin_status(lib, M=0) == _lib.OK
    assert packin_status(lib, w=packed(rows=0, q=0x40000)) == _lib.OK
    assert lib.convrot_linear_packin(A16C, _lib.BF16, 256, 1, None, None, 0, 0x90000, _lib.BF16, 64,
                                     None) == _lib.ERR_INVALID_ARG


def test_gated_packin_checks(lib):
    assert gated_packin_status(lib, fn=_lib.ACT_NONE) == _lib.ERR_INVALID_ARG
    assert gated_packin_status(lib, ydt=_lib.I32) == _lib.ERR_DTYPE
    assert gated_packin_status(lib, xdt=_lib.F32) == _lib.ERR_DTYPE
    assert gated_packin_status(lib, M=5) == _lib.ERR_INVALID_ARG
    k4112 = dict(K=4112, G=16)
    assert gated_packin_status(lib, gate=packed(rows=64, q=0x40000, **k4112),
                               up=packed(rows=64, q=0x80000, **k4112)) == _lib.ERR_INVALID_ARG
    assert gated_packin_status(lib, up=packed(rows=48, q=0x80000)) == _lib.ERR_MISMATCH
    assert gated_packin_status(lib, up=packed(rows=64, G=64, q=0x80000)) == _lib.ERR_MISMATCH
    tiled = packed(rows=64, q=0x80000, layout=_lib.LAYOUT_TILE16)
    assert gated_packin_status(lib, up=tiled) == _lib.ERR_INVALID_ARG
    assert b"same layout" in lib.convrot_last_error()
    assert gated_packin_status(lib, M=0) == _lib.OK
