"""Benchmark of the ConvRot W8A8 linear hot path on one MI355X.

A step is one pass of the whole path over one batch: pack the activation
rows once (rotate + absmax + int8), then run every linear that shares the
packed activation.  The default workload is the DiT attention projection:
X bf16 [4096, 3072] with 8 outlier channels, a fused QKV weight
[9216, 3072] and a second weight [3072, 3072], G = 256, bf16 output.  Weights
are packed once before timing (offline, as in a checkpoint).

Inputs live in HBM before timing starts.  To keep the 256 MB Infinity Cache
from serving them, each step uses the next of several independent buffer sets
(activations, packed weights, outputs) whose total exceeds 512 MB.

Prints one JSON line on stdout; per-kernel details go to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_I8_TOPS = 5000.0    # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0    # 8 TB/s HBM3E
COLD_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant GEMM from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when there is none for this
    workload or the GEMM source has changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_gemm_i8_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, "w8a8_int8_linear_amd", "csrc", "gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256") != digest:
        return None
    return int(fields["traffic_bytes"])


def make_workload(name: str):
    import workloads as W

    if name == "dit_attn_proj":
        return W.config2()
    if name == "dit_mlp":
        return W.config3()
    if name == "large_m_qkv":
        return W.config4(with_routed=False)
    if name.startswith("decode_m"):
        m = int(name[len("decode_m"):])
        return W.config5(M=m, G=64)
    if name == "unit_layer":
        return W.config1()
    raise SystemExit(f"unknown workload {name}")


class Kernels:
    """Device state for one buffer set plus the step itself."""

    def __init__(self, wl, dev, torch, cr, template=None):
        self.torch, self.cr = torch, cr
        xdt = torch.bfloat16 if wl.xdtype == "bf16" else torch.float32
        self.odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
        self.G = wl.G
        if template is None:
            self.X = torch.from_numpy(wl.X).to(xdt).to(dev)
            self.pw = []
            self.bias = []
            for lin in wl.linears:
                wd = torch.from_numpy(lin.W).to(torch.bfloat16 if lin.wdtype == "bf16" else torch.float32).to(dev)
                self.pw.append(cr.pack_weight(wd, wl.G))
                del wd
                self.bias.append(torch.from_numpy(lin.b).to(dev) if lin.b is not None else None)
        else:
            self.X = template.X.clone()
            self.pw = [cr.Packed(p.q.clone(), p.scale.clone(), p.group) for p in template.pw]
            self.bias = template.bias
        M, K = self.X.shape
        self.mlp = wl.extra.get("activation") == "gelu_erf"
        self.pa = cr.Packed(torch.empty((M, K), dtype=torch.int8, device=dev),
                            torch.empty(M, dtype=torch.float32, device=dev), wl.G)
        self.Y = [torch.empty((M, p.rows), dtype=self.odt, device=dev) for p in self.pw]
        if self.mlp:
            Kd = self.pw[0].rows
            self.pa2 = cr.Packed(torch.empty((M, Kd), dtype=torch.int8, device=dev),
                                 torch.empty(M, dtype=torch.float32, device=dev), wl.G)

    def nbytes(self):
        t = [self.X, self.pa.q, *[p.q for p in self.pw], *self.Y]
        if self.mlp:
            t.append(self.pa2.q)
        return sum(x.numel() * x.element_size() for x in t)

    def step(self, ev=None):
        cr = self.cr
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        cr.pack_act(self.X, self.G, out=self.pa)
        rec(1)
        if not self.mlp:
            for j, (p, b, y) in enumerate(zip(self.pw, self.bias, self.Y)):
                cr.linear(self.pa, p, b, out=y)
                rec(2 + j)
        else:
            cr.linear(self.pa, self.pw[0], self.bias[0], out=self.Y[0])
            rec(2)
            h = self.torch.nn.functional.gelu(self.Y[0])
            rec(3)
            cr.pack_act(h, self.G, out=self.pa2)
            rec(4)
            cr.linear(self.pa2, self.pw[1], self.bias[1], out=self.Y[1])
            rec(5)


def cpu_baseline(wl, budget_s: float = 15.0):
    """Time the oracle on a bounded row sample of the same step."""
    import threadpoolctl

    import oracle.convrot_oracle as O

    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    packed = []
    for lin in wl.linears:
        qw, sw, _ = O.pack(lin.W, wl.G)
        packed.append((qw, sw, lin.b))
    M, K = wl.X.shape
    ops_per_row = sum(2.0 * K * qw.shape[0] for qw, _, _ in packed) if not wl.extra.get("activation") == "gelu_erf" \
        else 2.0 * K * packed[0][0].shape[0] * 2

    def run(m):
        t0 = time.perf_counter()
        qx, sx, _ = O.pack(wl.X[:m], wl.G)
        for qw, sw, b in packed[:1] if wl.extra.get("activation") == "gelu_erf" else packed:
            O.epilogue64(O.int_gemm(qx, qw), sx, sw, b).astype(np.float32)
        return time.perf_counter() - t0

    m = min(M, 64)
    t = run(m)
    while m < M and t < budget_s / 4:
        m = min(M, m * 4)
        t = run(m)
    return {"value": round(ops_per_row * m / t / 1e12, 6), "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"first {m} of {M} activation rows of the same step (pack + every linear's exact int GEMM "
                      f"and epilogue; weights packed beforehand, untimed); {t:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_attn_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is data parallel over rows "
              "and multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    import w8a8_int8_linear_amd as cr

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    t0 = time.time()
    wl = make_workload(args.workload)
    log(f"[bench] workload {wl.name}: X {wl.X.shape} {wl.xdtype}, linears "
        f"{[(l.name, l.W.shape) for l in wl.linears]}, G={wl.G} (inputs {time.time() - t0:.1f}s)")

    sets = [Kernels(wl, dev, torch, cr)]
    while sum(s.nbytes() for s in sets) < COLD_BYTES:
        sets.append(Kernels(wl, dev, torch, cr, template=sets[0]))
    log(f"[bench] {len(sets)} buffer sets, {sum(s.nbytes() for s in sets) / 2**20:.0f} MiB rotated per cycle")
    torch.cuda.synchronize()

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        sets[i % len(sets)].step()
    torch.cuda.synchronize()

    n_ev = 2 + len(wl.linears) + (2 if wl.extra.get("activation") == "gelu_erf" else 0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        sets[i % len(sets)].step(evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1e3 / args.steps

    dur = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(n_ev - 1)] for i in range(args.steps)])
    avg_ms = dur.mean(axis=0)
    M, K = wl.X.shape
    in_b = 2 if wl.xdtype == "bf16" else 4
    out_b = 2 if wl.out_dtype == "bf16" else 4
    kernels = {}
    pack_bytes = M * K * (in_b + 1) + 4 * M
    kernels["pack_act"] = {"us": avg_ms[0] * 1e3, "GB/s": pack_bytes / (avg_ms[0] * 1e-3) / 1e9}
    kernels["pack_act"]["frac_hbm"] = kernels["pack_act"]["GB/s"] / PEAK_HBM_GBS
    total_ops = 0.0
    lin_names = [l.name for l in wl.linears]
    if wl.extra.get("activation") == "gelu_erf":
        slots = {lin_names[0]: 1, "gelu": 2, "pack_act2": 3, lin_names[1]: 4}
    else:
        slots = {n: 1 + j for j, n in enumerate(lin_names)}
    for j, lin in enumerate(wl.linears):
        N, Kw = lin.W.shape
        ops = 2.0 * M * N * Kw
        total_ops += ops
        t = avg_ms[slots[lin.name]] * 1e-3
        gemm_bytes = M * Kw + 4 * M + N * Kw + 8 * N + M * N * out_b
        kernels[f"linear_{lin.name}"] = {"us": t * 1e6, "TOPS": ops / t / 1e12, "frac_mfma": ops / t / 1e12 / PEAK_I8_TOPS,
                                         "GB/s": gemm_bytes / t / 1e9, "M": M, "N": N, "K": Kw}
    if "gelu" in slots:
        kernels["gelu_torch"] = {"us": avg_ms[slots["gelu"]] * 1e3}
        Kd = wl.linears[0].W.shape[0]
        t = avg_ms[slots["pack_act2"]] * 1e-3
        kernels["pack_act2"] = {"us": t * 1e6, "GB/s": (M * Kd * 3 + 4 * M) / t / 1e9}
    for k, v in kernels.items():
        log(f"[bench] {k}: " + ", ".join(f"{a}={b:.4g}" if isinstance(b, float) else f"{a}={b}" for a, b in v.items()))

    # Dominant kernel: the largest linear.
    big = max(wl.linears, key=lambda l: l.W.shape[0] * l.W.shape[1])
    kb = kernels[f"linear_{big.name}"]
    small_m = M <= 16
    if small_m:
        roof = {"kernel": f"linear_{big.name}", "bound": "hbm", "achieved": round(kb["GB/s"], 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(kb["GB/s"] / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"kernel": f"linear_{big.name}", "bound": "mfma", "achieved": round(kb["TOPS"], 2),
                "peak": PEAK_I8_TOPS, "unit": "TFLOP/s", "frac": round(kb["TOPS"] / PEAK_I8_TOPS, 4),
                "traffic": measured_traffic(args.workload)}

    value = total_ops / (ms_step * 1e-3) / 1e12
    result = {
        "metric": "convrot_linear effective int8 TOPS + % MFMA peak; rotate+quant GB/s % HBM",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded; shapes and outlier structure of the workload, no checkpoint)",
        "config": {"workload": wl.name, "M": M, "K": K, "N": [l.W.shape[0] for l in wl.linears], "G": wl.G,
                   "in": wl.xdtype, "out": wl.out_dtype, "buffer_sets": len(sets)},
        "roofline": roof,
        "pack_roofline": {"bound": "hbm", "achieved": round(kernels["pack_act"]["GB/s"], 2), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(kernels["pack_act"]["frac_hbm"], 4)},
        "kernels_us": {k: round(v["us"], 3) for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
