"""Build the HIP libraries in-tree for gfx950 with hipcc: libconvrot.so (the
linear layer, include/convrot.h) and libconvrot_probe.so (hardware
measurement probes used by bench.py, include/convrot_probe.h).

Usage: python -m w8a8_int8_linear_amd.build   (or call build()).
Objects go to <repo>/_build/, the shared libraries next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_NAME = "libconvrot.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
SOURCES = ["api.cpp", "pack_rows.hip", "gemm_i8.hip", "gemm_bf16.hip", "gemm_act.hip", "gemm_gated.hip", "gemv.hip",
           "w4.hip", "smooth.hip", "lora.hip", "tile.hip"]
PROBE_NAME = "libconvrot_probe.so"
PROBE_PATH = os.path.join(PKG_DIR, PROBE_NAME)
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 arithmetic stays off in all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # Every kernel must have its host launch stub: a kernel body the host pass
    # cannot type-check is silently left without one.
    r = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l for l in r.stdout.splitlines() if "convrot" in l]
    if r.returncode != 0 or missing:
        raise RuntimeError(f"{os.path.basename(path)} has undefined symbols:\n" + "\n".join(missing[:20]))
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libconvrot.so and
    libconvrot_probe.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, os.cpu_count() or 2))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
