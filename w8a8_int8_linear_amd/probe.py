"""Hardware measurement probes (libconvrot_probe.so, include/convrot_probe.h).

``mfma_i8(device)`` runs the MFMA-only int8 loop on random codes (normal,
sigma 32 code units) with one workgroup per CU and returns the rate it reached and the shader clock each
CU ran at during it (from the s_memtime / s_memrealtime counters the kernel
stamps).  ``copy_gbps(device)`` times a plain device-to-device copy.  These
are the measured ceilings next to which bench.py reports the published peaks;
they are not part of the linear layer.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvrot_probe.so")
THREADS = 512
CHAINS = 8
OPS_PER_MFMA = 32768
REALTIME_HZ = 100e6   # s_memrealtime counts at a constant 100 MHz
EXPORTED = ("convrot_probe_copy", "convrot_probe_mfma_i8", "convrot_probe_read")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise ImportError(f"{PROBE_PATH} is missing: build it with `python -m w8a8_int8_linear_amd.build`")
        lib = ctypes.CDLL(PROBE_PATH)
        vp = ctypes.c_void_p
        lib.convrot_probe_mfma_i8.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp]
        lib.convrot_probe_mfma_i8.restype = ctypes.c_int
        lib.convrot_probe_copy.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, vp]
        lib.convrot_probe_copy.restype = ctypes.c_int
        lib.convrot_probe_read.argtypes = [vp, ctypes.c_int64, ctypes.c_int, vp, ctypes.c_int, vp]
        lib.convrot_probe_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def mfma_i8(device: torch.device, iters: int = 20000, seed: int = 7) -> dict:
    """int8 MFMA-only throughput (TOPS) over one workgroup per CU, and the
    per-CU shader clock (GHz: median, min, max) during the loop."""
    lib = load()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    g = torch.Generator(device="cpu").manual_seed(seed)
    # codes like those of a quantised normal row (row max about 4 sigma, so
    # sigma is about 32 code units), as the layer's GEMM multiplies
    z = torch.randn(cus * THREADS * 64, generator=g) * 32.0
    ops_bytes = z.round().clamp(-127, 127).to(torch.int8).to(device)
    stamps = torch.zeros(cus * 4, dtype=torch.int64, device=device)
    sink = torch.empty(cus * THREADS, dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream(device)

    def run(n):
        st = lib.convrot_probe_mfma_i8(ops_bytes.data_ptr(), cus, n, stamps.data_ptr(), sink.data_ptr(), 0,
                                       stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"convrot_probe_mfma_i8 failed ({st})")

    run(max(1, iters // 10))  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(iters)
    e1.record(stream)
    torch.cuda.synchronize(device)
    ms = e0.elapsed_time(e1)
    s = stamps.view(cus, 4).cpu().numpy().astype(np.float64)
    ghz = (s[:, 1] - s[:, 0]) / ((s[:, 3] - s[:, 2]) / REALTIME_HZ) / 1e9
    ops = cus * (THREADS // 64) * iters * CHAINS * OPS_PER_MFMA
    return {"TOPS": round(ops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3), "cus": cus,
            "sclk_GHz": round(float(np.median(ghz)), 3), "sclk_GHz_min": round(float(ghz.min()), 3),
            "sclk_GHz_max": round(float(ghz.max()), 3)}


def copy_gbps(device: torch.device, mib: int = 1024, reps: int = 5) -> dict:
    """A device-to-device copy of ``mib`` MiB, read + write bytes per second
    (median over ``reps``): the streaming probe kernel at several grid sizes
    (the best is the measured streaming ceiling) and torch's own copy."""
    lib = load()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    nbytes = mib << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(device)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize(device)
            ts.append(e0.elapsed_time(e1))
        return round(2 * nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)

    def probe(grid):
        def run():
            if lib.convrot_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid, stream.cuda_stream) != 0:
                raise RuntimeError("convrot_probe_copy failed")
        return run

    by_grid = {f"{k}x": timed(probe(k * cus)) for k in (4, 8, 16)}
    out = {"GBps": max(by_grid.values()), "by_grid_per_cu": by_grid, "torch_copy_GBps": timed(lambda: dst.copy_(src))}
    del src, dst
    return out


def _sweep(device, sizes_mib, span_mib, reps, reads_only):
    lib = load()
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    span = span_mib << 20
    src = torch.ones(span, dtype=torch.uint8, device=device)
    dst = None if reads_only else torch.empty_like(src)
    sink = torch.empty(8 * cus * 256, dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream(device)
    pts = []
    for mib in sizes_mib:
        nb = mib << 20
        slots = max(1, span // nb)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream(device).cuda_stream
            for r in range(reps):
                off = (r % slots) * nb
                if reads_only:
                    st = lib.convrot_probe_read(src.data_ptr() + off, nb, 8 * cus, sink.data_ptr(), 0, cs)
                else:
                    st = lib.convrot_probe_copy(src.data_ptr() + off, dst.data_ptr() + off, nb, 8 * cus, cs)
                if st != 0:
                    raise RuntimeError("probe launch failed")
        g.replay()
        torch.cuda.synchronize(device)
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize(device)
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        pts.append(((1.0 if reads_only else 2.0) * nb, float(np.median(ts))))
        del g
    x = np.array([p[0] for p in pts])
    y = np.array([p[1] for p in pts])
    slope, t0 = np.polyfit(x, y, 1)
    del src, dst
    return {"t0_us": round(float(t0), 3), "GBps": round(1e-3 / float(slope), 1),
            "points_us": {f"{mib}MiB": round(t, 2) for mib, (_, t) in zip(sizes_mib, pts)}}


def copy_sweep(device: torch.device, sizes_mib=(4, 16, 64, 256), span_mib: int = 1024, reps: int = 16) -> dict:
    """Streaming-copy time against size, each size copied ``reps`` times in
    one HIP graph over consecutive slices of a ``span_mib`` buffer (so the
    256 MB Infinity Cache cannot serve repeats) and timed with events: the
    per-launch fixed cost t0 and the streaming bandwidth of the least-squares
    fit t = t0 + (read + write bytes) / BW.  A kernel moving B bytes cannot
    beat t0 + B / BW on this GPU."""
    return _sweep(device, sizes_mib, span_mib, reps, reads_only=False)


def read_sweep(device: torch.device, sizes_mib=(4, 8, 16, 64, 256), span_mib: int = 1024, reps: int = 16) -> dict:
    """The same fit for a streaming read with no stores, t = t0 + bytes / BW:
    the floor of a read-dominated launch such as small-M weight streaming."""
    return _sweep(device, sizes_mib, span_mib, reps, reads_only=True)
