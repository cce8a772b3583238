"""Compiled-code check (CPU only): no instruction of any gfx950 kernel touches
a vector register that an outstanding LDS read still has to write.

Every HIP source of the library is compiled to device assembly with the
build's own flags, and every kernel in it is scanned (tests/isa_scan.py).
The scanner itself is pinned first on small hand-written snippets: a
planted hazard must be found, and the same code with the wait in place
must pass.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

import pytest

import isa_scan

from w8a8_int8_linear_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def _kernel(body: str) -> str:
    return "demo_kernel:                ; @demo_kernel\n" + body + "\n"


def test_scanner_finds_a_planted_hazard():
    asm = _kernel("""
        ds_read_b128 v[4:7], v1
        v_add_u32_e32 v5, 1, v2
        s_waitcnt lgkmcnt(0)
        s_endpgm""")
    (rep,) = isa_scan.scan_asm(asm)
    assert len(rep.hazards) == 1 and rep.hazards[0][1] == [5]


def test_scanner_accepts_the_waited_version():
    asm = _kernel("""
        ds_read_b128 v[4:7], v1
        s_waitcnt lgkmcnt(0)
        v_add_u32_e32 v5, 1, v2
        s_endpgm""")
    (rep,) = isa_scan.scan_asm(asm)
    assert rep.hazards == []


def test_scanner_follows_branches_and_partial_waits():
    # The read into v8 is still owed on the taken branch after a wait that
    # retires only the older read; the join must carry it to the use.
    asm = _kernel("""
        ds_read_b32 v2, v1
        ds_read_b32 v8, v1
        s_cbranch_scc0 .LBB0_2
        s_waitcnt lgkmcnt(1)
        v_mov_b32_e32 v3, v2
.LBB0_2:
        v_mov_b32_e32 v9, v8
        s_waitcnt lgkmcnt(0)
        s_endpgm""")
    (rep,) = isa_scan.scan_asm(asm)
    assert [h[1] for h in rep.hazards] == [[8]]


def _compile(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [B.HIPCC, *B.COMMON_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-2000:]}")
    return out


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_compiled_kernels_have_no_lds_register_hazards(tmp_path):
    jobs = min(len(HIP_SOURCES), max(1, os.cpu_count() or 2))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda s: _compile(s, str(tmp_path)), HIP_SOURCES))
    bad = []
    kernels = 0
    for src, path in zip(HIP_SOURCES, outs):
        with open(path) as f:
            reports = isa_scan.scan_asm(f.read())
        kernels += len(reports)
        for rep in reports:
            if rep.hazards:
                bad.append(f"{src}: {rep.name}: {rep.hazards[:3]}")
    assert kernels > 50, "expected every kernel instantiation to be scanned"
    assert not bad, "LDS-read register hazards:\n" + "\n".join(bad)
