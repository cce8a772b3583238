"""Benchmark of the ConvRot W8A8 linear hot path on one MI355X.

A step is one pass of the whole path over one batch: pack the activation
rows once (rotate + absmax + int8), then run every linear that consumes the
packed activation; where a workload chains layers (the MLP pair, the gated
FFN) the intermediate activation is packed again.  Weights are packed once
before timing (offline, as in a checkpoint).  Layers whose input width is not
a multiple of G run on the routed bf16 linear.  The activation between chained
layers runs in the producing linear's epilogue (GELU after the MLP up
projection; gate and up as one gated launch); ``--unfused`` runs it as a
separate torch op after plain linears instead.

Workloads (``--workload``):
  large_m_qkv    (default) X bf16 [32700, 6144], 0.1% of entries x100;
                 W [18432, 6144]; plus the routed layer X' [32700, 2688] ->
                 W' [6144, 2688] on the bf16 linear (2688 % 256 != 0).
  dit_attn_proj  X bf16 [4096, 3072], 8 outlier channels; fused QKV
                 W [9216, 3072] and a second W [3072, 3072] share one pack.
                 Both run as one launch over the concatenated packed weight
                 (per-row packing makes it the concatenation of the two packed
                 weights), each output a column view of one buffer;
                 ``--separate-linears`` launches them one by one.
                 Suffix "_lora{r}": a rank-r adapter on the QKV layer, its
                 correction computed from the unrotated X and added to the
                 QKV output (two launches after the linear).
  dit_mlp        X bf16 [8192, 3072]; W_up [12288, 3072], GELU, W_down
                 [3072, 12288].
  decode_m{M}_g{G}[r]  gated FFN at M in {1, 4, 16}, K = 1152: W_gate, W_up
                 [6912, 1152] share one pack, h = gelu_tanh(gate) * up feeds
                 W_down [1152, 6912]; G in {16, 64, 1024}, "r" = randomized
                 block rotation (G = 128).  G = 1024 divides neither width,
                 so every linear routes to bf16.  Suffix "_w4": the same layer
                 with int4 weights (W4A8; codes in [-7, 7], nibble pairs).
                 Weights and packed activations take the TILE16 layout
                 (``--row-weights`` / ``--row-activations`` keep rows).
  unit_layer     X fp32 [64, 1024], W [1024, 1024], fp32 output.

Inputs live in HBM before timing starts.  To keep the 256 MB Infinity Cache
from serving them, each step uses the next of several independent buffer sets
(activations, packed weights, outputs) whose total exceeds 512 MB.

The step is captured as HIP graphs of exactly K and of 2K steps (the launches
a serving loop would capture).  Each graph is replayed three times, each
replay bracketed by device synchronisation, and the median taken.  A replay
carries a fixed cost (the graph launch and the ramp of its first kernel)
besides its steps, so ``ms_per_step`` is the slope between the two lengths,
(t_2K - t_K) / K, which does not depend on K; the K-step replay divided by K
is reported as ``ms_per_step_k_graph``.  Per-launch durations come from one
graph per launch of the step, holding that launch repeated over the buffer
sets, timed with events on its stream and divided by the repeat count.
``--eager`` launches every kernel from Python instead, with an event between
consecutive launches (at decode sizes that measures the host's launch cost).

Besides the published peaks the line carries measured ceilings of the GPU it
ran on: a device copy's GB/s, the fixed cost and bandwidth of streaming
copies and reads fitted over sizes, and the int8 MFMA rate and shader clock
of an MFMA-only loop on random operands (libconvrot_probe.so).

Prints one JSON line on stdout; per-kernel details go to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
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
SMALL_M = 16             # up to this many rows a linear runs on the weight-streaming kernel
PACKIN_GATED_ROWS = 4    # with --packin, up to this many decode rows the gated launch packs its own input
METRIC = "convrot_linear effective int8 TOPS + % MFMA peak; rotate+quant GB/s % HBM"
# the sources each kernel is compiled from; a traffic summary is valid only for these exact bytes
KERNEL_SOURCE = {
    "gemm_i8": ("gemm_kernel.h", "gemm_pp.h", "lanes.h", "epilogue.h", "gemm_i8.hip"),
    "gemm_i8_act": ("gemm_kernel.h", "gemm_pp.h", "lanes.h", "epilogue.h", "gemm_act.hip"),
    "gemm_i8_gated": ("gemm_kernel.h", "epilogue.h", "gemm_gated.hip"),
    "gemm_bf16": ("gemm_kernel.h", "gemm_pp.h", "lanes.h", "epilogue.h", "gemm_bf16.hip"),
    "gemv_i8": ("gemv.hip", "epilogue.h", "w4_codec.h", "pack_core.h", "lanes.h"),
    "gemv_w4": ("gemv.hip", "epilogue.h", "w4_codec.h", "pack_core.h", "lanes.h"),
    "pack_rows": ("pack_rows.hip", "pack_core.h", "lanes.h"),
}


def _code_only(text: str) -> str:
    """A source file's code without its comments and blank space, so that an
    edit of the prose alone does not invalidate counters taken on the same
    kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())


def source_digest(kernel: str) -> str:
    """sha256 of the code (comments and blank space removed) of the sources a
    kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCE[kernel]:
        with open(os.path.join(ROOT, "w8a8_int8_linear_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when there is none for this
    workload or the kernel's source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCE:
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_digest(kernel):
        return None
    return int(fields["traffic_bytes"])


def make_workload(name: str):
    import workloads as W

    if name == "dit_attn_proj":
        return W.config2()
    m = re.fullmatch(r"dit_attn_proj_lora(\d+)", name)
    if m:
        wl = W.config2()
        wl.name += f"_lora{m.group(1)}"
        wl.extra["lora_rank"] = int(m.group(1))
        return wl
    if name == "dit_mlp":
        return W.config3()
    if name == "large_m_qkv":
        return W.config4(with_routed=True)
    m = re.fullmatch(r"decode_m(\d+)_g(\d+)(r?)(_w4)?", name)
    if m:
        wl = W.config5(M=int(m.group(1)), G=int(m.group(2)), kind="randomized" if m.group(3) else "regular")
        if m.group(4):
            wl.name += "_w4"
            wl.extra["wbits"] = 4
        return wl
    if name == "unit_layer":
        return W.config1()
    raise SystemExit(f"unknown workload {name}")


class Op:
    """One timed launch of the step and what it moves or computes."""

    def __init__(self, name, fn, kind, M=0, N=0, K=0, in_b=0, out_b=0, epilogue="", packin=False):
        self.name, self.fn, self.kind = name, fn, kind
        self.M, self.N, self.K, self.in_b, self.out_b = M, N, K, in_b, out_b
        # a linear that packs its own activation rows: reads X (in_b bytes per
        # element) instead of the int8 codes and scales
        self.packin = packin
        # "" plain, "act" activation in the epilogue, "gated" act(gate) * up:
        # N output columns from 2N weight rows
        self.epilogue = epilogue
        self.epilogue_rank = 0  # LoRA rank of a "lora" launch

    @property
    def kernel(self):
        if self.kind == "pack":
            return "pack_rows"
        if self.kind in ("int8", "int4"):
            if self.M <= SMALL_M:
                return "gemv_i8" if self.kind == "int8" else "gemv_w4"
            return "gemm_i8" + (f"_{self.epilogue}" if self.epilogue else "")
        if self.kind == "bf16":
            return "gemm_bf16"
        if self.kind == "lora":
            return "lora"
        return "torch"

    @property
    def rows(self):
        """weight rows the launch contracts against"""
        return 2 * self.N if self.epilogue == "gated" else self.N

    def ops(self):
        return 2.0 * self.M * self.rows * self.K if self.kind in ("int8", "int4", "bf16") else 0.0

    def bytes(self):
        M, N, K = self.M, self.N, self.K
        if self.kind == "pack":
            return M * K * (self.in_b + 1) + 4 * M
        if self.kind in ("int8", "int4"):
            R = self.rows
            wb = R * K if self.kind == "int8" else R * K // 2  # int4: two codes per byte
            xb = M * K * self.in_b if self.packin else M * K + 4 * M
            return xb + wb + 8 * R + M * N * self.out_b
        if self.kind == "bf16":
            return 2 * M * K + 2 * N * K + 4 * N + M * N * self.out_b
        if self.kind == "lora":
            # X and A read, T written and read, B read, Y read and written (K here is the rank's input width)
            r = self.epilogue_rank
            return 2 * M * K + 2 * r * K + 4 * M * r + 2 * N * r + 2 * M * N * self.out_b
        return 0


class StepSet:
    """Device state of one buffer set and the ordered launches of one step."""

    def __init__(self, wl, dev, torch, cr, template=None, fused=True, merge=True, producer_fusion=False,
                 tiled=False, packin=False, xtiled=False):
        self.torch, self.cr, self.wl, self.fused = torch, cr, wl, fused
        # --packin, decode with at most PACKIN_GATED_ROWS rows and int8
        # weights: the gated launch packs its own bf16 input rows (the down
        # projection, whose 16-wave workgroups would each pack a 6912-wide
        # row, keeps the separate pack).  Off by default: with TILE16
        # weights the separate pack measured level at one row and faster
        # from two rows on.
        self.packin = (packin and fused and wl.cfg == 5 and wl.X.shape[0] <= PACKIN_GATED_ROWS
                       and wl.xdtype == "bf16" and wl.extra.get("wbits") != 4
                       and all(l.W.shape[1] % wl.G == 0 for l in wl.linears))
        self.producer_fusion = producer_fusion and fused and wl.cfg == 3
        # weights in the TILE16 layout, which only the M <= 16 path reads
        self.tiled = tiled and wl.X.shape[0] <= 16
        # packed activations in the TILE16 layout (M <= 16, int8 weights)
        self.xtiled = xtiled and wl.X.shape[0] <= 16 and wl.extra.get("wbits") != 4
        # linears that share the packed activation run as one launch over the
        # concatenated weight (configs whose linears all read the same input)
        self.merge = merge and wl.cfg == 2 and all(l.W.shape[1] % wl.G == 0 for l in wl.linears)
        bf16, f32 = torch.bfloat16, torch.float32
        self.xdt = bf16 if wl.xdtype == "bf16" else f32
        self.odt = bf16 if wl.out_dtype == "bf16" else f32
        G, kind = wl.G, wl.kind
        K0 = wl.X.shape[1]

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

        if template is None:
            self.signs = {}
            if wl.signs is not None:
                self.signs[K0] = up(wl.signs, torch.int8)
            if wl.extra.get("signs_down") is not None:
                sd = wl.extra["signs_down"]
                self.signs[sd.shape[0]] = up(sd, torch.int8)
            self.X = up(wl.X, self.xdt)
            self.W, self.b = {}, {}
            routed = wl.extra.get("routed")
            lins = list(wl.linears) + ([routed] if routed is not None else [])
            if self.merge:
                from workloads import Linear as _Lin
                cat = _Lin("_".join(l.name for l in wl.linears), np.concatenate([l.W for l in wl.linears]),
                           np.concatenate([l.b for l in wl.linears]) if all(l.b is not None for l in wl.linears)
                           else None, wl.linears[0].wdtype)
                lins = [cat]
            for lin in lins:
                K = lin.W.shape[1]
                wd = up(lin.W, bf16 if lin.wdtype == "bf16" else f32)
                if lin is routed or K % G != 0:
                    self.W[lin.name] = wd.to(bf16)
                elif wl.extra.get("wbits") == 4:
                    self.W[lin.name] = cr.pack_weight_w4(wd, G, kind, self.signs.get(K))
                    if self.tiled and lin.W.shape[0] % 16 == 0 and K % 128 == 0:
                        self.W[lin.name] = cr.tile_weight_w4(self.W[lin.name])
                else:
                    self.W[lin.name] = cr.pack_weight(wd, G, kind, self.signs.get(K))
                    if self.tiled and lin.W.shape[0] % 16 == 0 and K % 64 == 0:
                        self.W[lin.name] = cr.tile_weight(self.W[lin.name])
                    del wd
                self.b[lin.name] = up(lin.b, f32) if lin.b is not None else None
            self.X2 = up(wl.extra["X_routed"], bf16) if "X_routed" in wl.extra else None
            self.lora = None
            if wl.extra.get("lora_rank"):
                import workloads as Wmod
                qkv = wl.linears[0]
                A, Bm = Wmod.lora_adapter(qkv.W.shape[1], qkv.W.shape[0], wl.extra["lora_rank"])
                self.lora = (up(A, bf16), up(Bm, bf16))
        else:
            self.lora = template.lora
            self.signs = template.signs
            self.X = template.X.clone()
            self.W = {k: (cr.Packed(v.q.clone(), v.scale.clone(), v.group, v.kind, v.signs, v.layout)
                          if isinstance(v, cr.Packed) else
                          cr.PackedW4(v.q.clone(), v.scale.clone(), v.K, v.group, v.kind, v.signs, v.layout)
                          if isinstance(v, cr.PackedW4) else v.clone()) for k, v in template.W.items()}
            self.b = template.b
            self.X2 = template.X2.clone() if template.X2 is not None else None
        self.bufs = []
        self.packed_acts = []
        self.ops = self._plan(dev)

    def _quant(self, w):
        """A packed (int8 or int4) weight, as opposed to a routed bf16 tensor."""
        return isinstance(w, (self.cr.Packed, self.cr.PackedW4))

    def _workspace(self, kind, M, N, K, dev):
        """The workspace a linear call of ``kind`` uses (the small-M K split's
        partial sums, the int4 path's expanded weight above 16 rows), owned
        by this buffer set; None when the call needs none."""
        ws = self.cr.linear_workspace(kind, M, N, K, dev)
        if ws is not None:
            self.bufs.append(ws)
        return ws

    # -- buffers -----------------------------------------------------------
    def _packed(self, rows, K, dev):
        t = self.torch
        tile = self.xtiled and K % 64 == 0
        q = t.empty((16 if tile else rows, K), dtype=t.int8, device=dev)[:rows]
        p = self.cr.Packed(q, t.empty(rows, dtype=t.float32, device=dev), self.wl.G, self.wl.kind, self.signs.get(K),
                           self.cr.TILE16 if tile else self.cr.ROWS)
        self.bufs.append(p.q)
        self.packed_acts.append(p)
        return p

    def _out(self, name, rows, dev):
        w = self.W[name]
        N = w.rows if self._quant(w) else w.shape[0]
        y = self.torch.empty((rows, N), dtype=self.odt, device=dev)
        self.bufs.append(y)
        return y

    def nbytes(self):
        t = [self.X, *self.bufs] + ([self.X2] if self.X2 is not None else [])
        for v in self.W.values():
            t.append(v.q if self._quant(v) else v)
        return sum(x.numel() * x.element_size() for x in t)

    # -- launches ----------------------------------------------------------
    def _pack_op(self, name, src, dst):
        cr = self.cr
        M, K = src.shape
        return Op(name, lambda: cr.pack_act(src, dst.group, dst.kind, dst.signs, out=dst), "pack", M=M, K=K,
                  in_b=src.element_size())

    def _linear_op(self, name, src, y):
        """src is a packed activation (int8 path) or a bf16 tensor (routed layer)."""
        cr, w, b = self.cr, self.W[name], self.b[name]
        ob = y.element_size()
        if isinstance(w, cr.Packed):
            ws = self._workspace("plain", src.rows, w.rows, w.K, y.device)
            return Op(f"linear_{name}", lambda: cr.linear(src, w, b, out=y, workspace=ws), "int8", M=src.rows,
                      N=w.rows, K=w.K, out_b=ob)
        if isinstance(w, cr.PackedW4):
            ws = self._workspace("w4", src.rows, w.rows, w.K, y.device)
            return Op(f"linear_{name}", lambda: cr.linear_w4(src, w, b, out=y, workspace=ws), "int4", M=src.rows,
                      N=w.rows, K=w.K, out_b=ob)
        ws = self._workspace("bf16", src.shape[0], w.shape[0], w.shape[1], y.device)
        return Op(f"linear_{name}", lambda: cr.linear_bf16(src, w, b, out=y, workspace=ws), "bf16", M=src.shape[0],
                  N=w.shape[0], K=w.shape[1], out_b=ob)

    def _plan(self, dev):
        wl, torch = self.wl, self.torch
        gelu = torch._C._nn.gelu
        M, K = self.X.shape
        ops = []
        names = [l.name for l in wl.linears]
        first = "_".join(names) if self.merge else names[0]
        if self.packin:
            return self._plan_packin(dev)
        if self._quant(self.W[first]):
            src0 = self._packed(M, K, dev)
            ops.append(self._pack_op("pack_act", self.X, src0))
        else:
            src0 = self.X
        if self.merge:
            # one launch; each linear's output is a column view of its buffer
            n = "_".join(names)
            y = self._out(n, M, dev)
            ops.append(self._linear_op(n, src0, y))
            if self.lora is not None:
                A, Bm = self.lora
                r = A.shape[0]
                yq = y[:, :wl.linears[0].W.shape[0]]
                ws = torch.empty(self.cr.lora_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)
                self.bufs.append(ws)
                op = Op(f"lora_{names[0]}", lambda yq=yq, ws=ws: self.cr.lora_add(self.X, A, Bm, 0.5, yq, workspace=ws),
                        "lora", M=M, N=yq.shape[1], K=K, out_b=y.element_size())
                op.epilogue_rank = r
                ops.append(op)
        elif wl.cfg in (1, 2):
            for n in names:
                y = self._out(n, M, dev)
                ops.append(self._linear_op(n, src0, y))
                if self.lora is not None and n == names[0]:
                    A, Bm = self.lora
                    r = A.shape[0]
                    ws = torch.empty(self.cr.lora_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)
                    self.bufs.append(ws)
                    op = Op(f"lora_{n}", lambda y=y, ws=ws: self.cr.lora_add(self.X, A, Bm, 0.5, y, workspace=ws),
                            "lora", M=M, N=y.shape[1], K=K, out_b=y.element_size())
                    op.epilogue_rank = r
                    ops.append(op)
        elif wl.cfg == 3 and self.producer_fusion:
            # GELU in the up projection's epilogue, which also emits the group
            # maxima of its rotated output; the down layer's pack takes its row
            # maxima from them
            h = self._out("up", M, dev)
            w, b = self.W["up"], self.b["up"]
            pm = torch.empty((M, w.rows // wl.G), dtype=torch.float32, device=dev)
            self.bufs.append(pm)
            ops.append(Op("linear_up_gelu_rowmax", lambda: self.cr.linear_act_rowmax(
                src0, w, wl.G, b, self.cr.GELU_ERF, out=h, rowmax=pm), "int8", M=M, N=w.rows, K=w.K,
                out_b=h.element_size(), epilogue="act"))
            pa2 = self._packed(M, h.shape[1], dev)
            ops.append(Op("pack_act2_rowmax", lambda: self.cr.pack_act_rowmax(h, pm, wl.G, out=pa2), "pack", M=M,
                          K=h.shape[1], in_b=h.element_size()))
            ops.append(self._linear_op("down", pa2, self._out("down", M, dev)))
        elif wl.cfg == 3:
            if self.fused:
                # GELU in the up projection's epilogue
                h = self._out("up", M, dev)
                w, b = self.W["up"], self.b["up"]
                wsa = self._workspace("plain", M, w.rows, w.K, dev)
                ops.append(Op("linear_up_gelu", lambda: self.cr.linear_act(src0, w, b, self.cr.GELU_ERF, out=h,
                                                                           workspace=wsa),
                              "int8", M=M, N=w.rows, K=w.K, out_b=h.element_size(), epilogue="act"))
            else:
                y_up = self._out("up", M, dev)
                ops.append(self._linear_op("up", src0, y_up))
                h = torch.empty_like(y_up)
                self.bufs.append(h)
                ops.append(Op("gelu_torch", lambda: gelu(y_up, out=h), "torch"))
            pa2 = self._packed(M, h.shape[1], dev)
            ops.append(self._pack_op("pack_act2", h, pa2))
            ops.append(self._linear_op("down", pa2, self._out("down", M, dev)))
        elif wl.cfg == 4:
            ops.append(self._linear_op("qkv", src0, self._out("qkv", M, dev)))
            r = wl.extra["routed"].name
            ops.append(self._linear_op(r, self.X2, self._out(r, M, dev)))
        elif wl.cfg == 5:
            wg, wu = self.W["gate"], self.W["up"]
            if self.fused and isinstance(wg, self.cr.PackedW4) and isinstance(wu, self.cr.PackedW4):
                # int4 gate and up in one launch
                h = self._out("gate", M, dev)
                bg, bu = self.b["gate"], self.b["up"]
                ws = self._workspace("w4_gated", M, wg.rows, wg.K, dev)
                ops.append(Op("linear_gate_up", lambda: self.cr.linear_w4_gated(
                    src0, wg, wu, bg, bu, self.cr.GELU_TANH, out=h, workspace=ws),
                    "int4", M=M, N=wg.rows, K=wg.K, out_b=h.element_size(), epilogue="gated"))
            elif self.fused and isinstance(wg, self.cr.Packed) and isinstance(wu, self.cr.Packed):
                # gate and up in one launch, gelu_tanh(gate) * up in its epilogue
                h = self._out("gate", M, dev)
                bg, bu = self.b["gate"], self.b["up"]
                wsg = self._workspace("gated", M, wg.rows, wg.K, dev)
                ops.append(Op("linear_gate_up", lambda: self.cr.linear_gated(src0, wg, wu, bg, bu, self.cr.GELU_TANH,
                                                                               out=h, workspace=wsg),
                              "int8", M=M, N=wg.rows, K=wg.K, out_b=h.element_size(), epilogue="gated"))
            else:
                g = self._out("gate", M, dev)
                u = self._out("up", M, dev)
                ops.append(self._linear_op("gate", src0, g))
                ops.append(self._linear_op("up", src0, u))
                t, h = torch.empty_like(u), torch.empty_like(u)
                self.bufs += [t, h]
                ops.append(Op("gelu_tanh_mul_torch",
                              lambda: torch.mul(gelu(g, approximate="tanh", out=t), u, out=h), "torch"))
            if self._quant(self.W["down"]):
                pa2 = self._packed(M, h.shape[1], dev)
                ops.append(self._pack_op("pack_act2", h, pa2))
                ops.append(self._linear_op("down", pa2, self._out("down", M, dev)))
            else:
                ops.append(self._linear_op("down", h, self._out("down", M, dev)))
        else:
            raise SystemExit(f"no step plan for config {wl.cfg}")
        return ops

    def _plan_packin(self, dev):
        """Decode step in three launches: gate and up with the pack of X in
        one, then the pack of h and the down projection."""
        cr = self.cr
        M = self.X.shape[0]
        wg, wu = self.W["gate"], self.W["up"]
        bg, bu = self.b["gate"], self.b["up"]
        h = self._out("gate", M, dev)
        ops = [Op("linear_gate_up", lambda: cr.linear_gated_packin(self.X, wg, wu, bg, bu, cr.GELU_TANH, out=h),
                  "int8", M=M, N=wg.rows, K=wg.K, in_b=self.X.element_size(), out_b=h.element_size(),
                  epilogue="gated", packin=True)]
        pa2 = self._packed(M, h.shape[1], dev)
        ops.append(self._pack_op("pack_act2", h, pa2))
        ops.append(self._linear_op("down", pa2, self._out("down", M, dev)))
        return ops

    def step(self, ev=None):
        if ev is None:
            for op in self.ops:
                op.fn()
            return
        ev[0].record()
        for i, op in enumerate(self.ops):
            op.fn()
            ev[i + 1].record()


def _gelu_erf(y):
    from scipy.special import erf

    return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))


def _gelu_tanh(y):
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))


def cpu_baseline(wl, budget_s: float = 12.0):
    """Time the oracle on a bounded row sample of the same step, with the
    pack (rotation + quantisation) and the quantised linears (exact integer
    GEMM + epilogue) timed separately.

    The oracle runs on every host core this process may use
    (``os.sched_getaffinity``), with the BLAS thread pool set to that count.
    Weights are packed beforehand (untimed).  Routed layers (fp64 linear) and
    the harness activations between chained layers (GELU in numpy) are timed
    as "other".
    """
    import threadpoolctl

    import oracle.convrot_oracle as O

    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        return _cpu_baseline(wl, budget_s, cores, O)


def _cpu_baseline(wl, budget_s, cores, O):
    G, kind = wl.G, wl.kind
    signs = {wl.X.shape[1]: wl.signs}
    if wl.extra.get("signs_down") is not None:
        signs[wl.extra["signs_down"].shape[0]] = wl.extra["signs_down"]
    routed = wl.extra.get("routed")
    lin = {l.name: l for l in wl.linears}
    if routed is not None:
        lin[routed.name] = routed

    def sg(K):
        return signs.get(K) if kind == "randomized" else None

    w4 = wl.extra.get("wbits") == 4
    packed = {}
    for n, l in lin.items():
        K = l.W.shape[1]
        if l is not routed and K % G == 0:
            if w4:
                nib, s, _, _ = O.pack_weight_int4(l.W, G, kind, sg(K))
                packed[n] = (O.unpack_nibbles(nib), s)
            else:
                q, s, _ = O.pack(l.W, G, kind, sg(K))
                packed[n] = (q, s)

    spent = {"pack": 0.0, "gemm": 0.0, "other": 0.0}
    work = {"pack_bytes": 0.0, "gemm_ops": 0.0}

    def timed(key, fn, *a):
        t0 = time.perf_counter()
        r = fn(*a)
        spent[key] += time.perf_counter() - t0
        return r

    def pack(x):
        work["pack_bytes"] += x.shape[0] * x.shape[1] * (2 if wl.xdtype == "bf16" else 4) + x.size + 4 * x.shape[0]
        qx, sx, _ = timed("pack", O.pack, x, G, kind, sg(x.shape[1]))
        return qx, sx

    def gemm(name, qx, sx):
        q, s = packed[name]
        work["gemm_ops"] += 2.0 * qx.shape[0] * q.shape[0] * q.shape[1]
        return timed("gemm", lambda: O.epilogue64(O.int_gemm(qx, q), sx, s, lin[name].b).astype(np.float32))

    def layer(name, x):
        if name in packed:
            return gemm(name, *pack(x))
        return timed("other", lambda: O.linear_unquantized64(x, lin[name].W, lin[name].b).astype(np.float32))

    def shared(names, x):
        if all(n in packed for n in names):
            qx, sx = pack(x)
            return [gemm(n, qx, sx) for n in names]
        return [layer(n, x) for n in names]

    adapter = None
    if wl.extra.get("lora_rank"):
        import workloads as Wmod
        qkv = wl.linears[0]
        adapter = Wmod.lora_adapter(qkv.W.shape[1], qkv.W.shape[0], wl.extra["lora_rank"])

    def run(m):
        t0 = time.perf_counter()
        x = wl.X[:m]
        if wl.cfg in (1, 2):
            ys = shared(list(l.name for l in wl.linears), x)
            if adapter is not None:
                ys[0] = ys[0] + timed("other", lambda: O.lora_delta64(x, adapter[0], adapter[1], 0.5)
                                      .astype(np.float32))
        elif wl.cfg == 3:
            h = timed("other", lambda y: _gelu_erf(y).astype(np.float32), layer("up", x))
            layer("down", h)
        elif wl.cfg == 4:
            layer("qkv", x)
            layer(routed.name, wl.extra["X_routed"][:m])
        elif wl.cfg == 5:
            g, u = shared(["gate", "up"], x)
            layer("down", timed("other", lambda: (_gelu_tanh(g) * u).astype(np.float32)))
        return time.perf_counter() - t0

    ops_per_row = sum(2.0 * l.W.shape[0] * l.W.shape[1] for l in lin.values())
    M = wl.X.shape[0]
    m = min(M, 64)
    t = run(m)
    while m < M and t < budget_s / 2:
        m = min(M, m * 4)
        for k in spent:
            spent[k] = 0.0
        for k in work:
            work[k] = 0.0
        t = run(m)
    reps, total = 1, t
    while total < budget_s and m == M:
        total += run(m)
        reps += 1
    out = {"value": round(ops_per_row * m * reps / total / 1e12, 6), "unit": "TOPS", "cores": int(cores),
           "kind": "oracle",
           "sample": f"first {m} of {M} activation rows of the same step, {reps} run(s) (pack + every linear's "
                     f"exact int GEMM and epilogue, routed layers in fp64, GELU in numpy; weights packed "
                     f"beforehand, untimed); {total:.2f} s on {cores} cores (BLAS threads = cores)",
           "seconds": {k: round(v, 3) for k, v in spent.items()}}
    if spent["pack"] > 0:
        out["pack_GBps"] = round(work["pack_bytes"] / spent["pack"] / 1e9, 4)
    if spent["gemm"] > 0:
        out["gemm_TOPS"] = round(work["gemm_ops"] / spent["gemm"] / 1e12, 6)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_m_qkv")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python in the timed region instead of replaying a captured graph")
    ap.add_argument("--unfused", action="store_true",
                    help="run the activation between chained layers as a separate torch op instead of in the "
                         "linear's epilogue")
    ap.add_argument("--producer-fusion", action="store_true",
                    help="MLP: the up projection's epilogue emits the rotated group maxima of its output and the "
                         "down layer's pack takes its row maxima from them")
    ap.add_argument("--separate-linears", action="store_true",
                    help="launch linears that share one packed activation one by one instead of as one launch over "
                         "the concatenated weight")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (calibrates HBM byte counters)")
    ap.add_argument("--row-weights", action="store_true",
                    help="decode (M <= 16): keep the packed weights in the row layout instead of the TILE16 layout "
                         "the weight-streaming kernel reads fastest")
    ap.add_argument("--row-activations", action="store_true",
                    help="decode (M <= 16): pack the activations in the row layout instead of the TILE16 layout "
                         "(one 16-row tile) that the weight-streaming kernel reads in whole cache lines")
    ap.add_argument("--packin", action="store_true",
                    help="decode with at most 4 rows: pack the gated launch's input inside the gated launch instead "
                         "of in a launch of its own")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured copy and MFMA-only ceilings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer is data parallel over "
              "rows, so each GPU runs the same one-GPU step on its own rows, and this library has no multi-GPU "
              "driver.", file=sys.stderr)
        sys.exit(2)

    import torch

    import w8a8_int8_linear_amd as cr

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    t0 = time.time()
    wl = make_workload(args.workload)
    log(f"[bench] workload {wl.name}: X {wl.X.shape} {wl.xdtype}, linears "
        f"{[(l.name, l.W.shape) for l in wl.linears]}, G={wl.G} {wl.kind} (inputs {time.time() - t0:.1f}s)")

    fused = not args.unfused
    merge = not args.separate_linears
    pf = args.producer_fusion
    tl = not args.row_weights
    pin = args.packin
    xtl = not args.row_activations
    sets = [StepSet(wl, dev, torch, cr, fused=fused, merge=merge, producer_fusion=pf, tiled=tl, packin=pin,
                    xtiled=xtl)]
    while sum(s.nbytes() for s in sets) < COLD_BYTES:
        sets.append(StepSet(wl, dev, torch, cr, template=sets[0], fused=fused, merge=merge, producer_fusion=pf,
                            tiled=tl, packin=pin, xtiled=xtl))
    ops = sets[0].ops
    log(f"[bench] {len(sets)} buffer sets, {sum(s.nbytes() for s in sets) / 2**20:.0f} MiB rotated per cycle; "
        f"launches: {[o.name for o in ops]}")
    torch.cuda.synchronize()

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        sets[i % len(sets)].step()
    torch.cuda.synchronize()

    n_ev = len(ops) + 1
    if args.eager:
        # Every launch from Python, an event between consecutive launches.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            sets[i % len(sets)].step(evs[i])
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start
    else:
        # K steps and 2K steps (cycling through the buffer sets) are captured
        # as HIP graphs and replayed: the kernels run back to back, without
        # the host's per-launch cost between them.  Each graph is replayed
        # once untimed, then three times timed (each replay bracketed by
        # device synchronisation); the medians give the per-step slope.
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    sets[i % len(sets)].step()
            g.replay()
            torch.cuda.synchronize()
            return g

        def replay_s(g, n=3):
            ts = []
            for _ in range(n):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                g.replay()
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
            return float(np.median(ts))

        g_k = capture(args.steps)
        t_k = replay_s(g_k)
        g_2k = capture(2 * args.steps)
        t_2k = replay_s(g_2k)
        t_k = min(t_k, replay_s(g_k))  # again after the long graph: same clock state
        del g_2k
        t_total = t_2k - t_k     # K steps without the fixed per-replay cost
        ms_k_graph = t_k * 1e3 / args.steps
        # Per-launch durations (events cannot be recorded inside a captured
        # graph here): launch j of the step, repeated over the buffer sets in
        # one graph, between two events on the stream it runs on.
        reps = max(16, len(sets))
        per_launch = []
        for j in range(len(ops)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(reps):
                    sets[r % len(sets)].ops[j].fn()
            g.replay()
            samples = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                samples.append(e0.elapsed_time(e1) / reps)
            per_launch.append(samples)
            del g
    ms_step = t_total * 1e3 / args.steps

    if args.eager:
        dur = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(n_ev - 1)]
                        for i in range(args.steps)])
    else:
        dur = np.array(per_launch).T  # [sample, launch]
    kernels = {}
    for j, op in enumerate(ops):
        us = dur[:, j] * 1e3
        t = us.mean() * 1e-6
        k = {"kernel": op.kernel, "us": us.mean(), "us_p10": np.percentile(us, 10), "us_p50": np.median(us),
             "us_p90": np.percentile(us, 90)}
        if op.bytes():
            k["GB/s"] = op.bytes() / t / 1e9
            k["frac_hbm"] = k["GB/s"] / PEAK_HBM_GBS
        if op.ops():
            k["TOPS"] = op.ops() / t / 1e12
            k["frac_mfma"] = k["TOPS"] / (PEAK_BF16_TFLOPS if op.kind == "bf16" else PEAK_I8_TOPS)
            k.update(M=op.M, N=op.rows, K=op.K)
        kernels[op.name] = k
    for k, v in kernels.items():
        log(f"[bench] {k}: " + ", ".join(f"{a}={b:.4g}" if isinstance(b, float) else f"{a}={b}" for a, b in v.items()))

    # Dominant kernel: the linear launch with the most algorithmic work
    # (weight bytes at decode sizes, ops otherwise); ties go to the earlier
    # launch, so the choice does not flip with timing noise.
    lin_ops = [op for op in ops if op.kind in ("int8", "int4", "bf16")]
    small = all(op.M <= SMALL_M for op in lin_ops)
    dom = max(lin_ops, key=lambda o: (o.bytes() if small else o.ops(), -ops.index(o)))
    kd = kernels[dom.name]
    if dom.M <= SMALL_M:
        roof = {"kernel": dom.kernel, "launch": dom.name, "bound": "hbm", "achieved": round(kd["GB/s"], 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kd["frac_hbm"], 4)}
    else:
        peak = PEAK_BF16_TFLOPS if dom.kind == "bf16" else PEAK_I8_TOPS
        roof = {"kernel": dom.kernel, "launch": dom.name, "bound": "mfma", "achieved": round(kd["TOPS"], 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(kd["TOPS"] / peak, 4)}
    roof["traffic"] = measured_traffic(dom.kernel, args.workload)

    value = sum(op.ops() for op in ops) / (ms_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "timing": "eager launches" if args.eager else
                  "slope between graphs of K and 2K steps, (t_2K - t_K) / K, medians of 3 replays",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if any(op.kind in ("int8", "int4") for op in ops) else "bf16",
        "data": "synthetic (seeded; shapes and outlier structure of the workload, no checkpoint)",
        "config": {"workload": wl.name, "M": wl.X.shape[0], "K": wl.X.shape[1],
                   "N": [l.W.shape[0] for l in wl.linears], "G": wl.G, "rotation": wl.kind, "in": wl.xdtype,
                   "epilogue": "fused" if fused else "separate", "launch": "eager" if args.eager else "graph",
                   "producer_fusion": bool(sets[0].producer_fusion),
                   "activation_pack": "in the gated launch" if sets[0].packin else "own launch",
                   "weight_layout": "tile16" if any(getattr(v, "layout", "rows") == "tile16"
                                                    for v in sets[0].W.values()) else "rows",
                   "activation_layout": "tile16" if any(getattr(o, "layout", "rows") == "tile16"
                                                        for o in sets[0].packed_acts) else "rows",
                   "shared_pack_linears": "one launch" if sets[0].merge else "one launch each",
                   "out": wl.out_dtype, "routed": [o.name for o in ops if o.kind == "bf16"],
                   "weights": "int4" if wl.extra.get("wbits") == 4 else "int8",
                   "buffer_sets": len(sets)},
        "roofline": roof,
        "kernels_us": {k: round(v["us"], 3) for k, v in kernels.items()},
    }
    packs = [op for op in ops if op.kind == "pack"]
    if packs:
        # the pack launch that takes the most time
        pk = max(packs, key=lambda o: kernels[o.name]["us"])
        kp = kernels[pk.name]
        result["pack_roofline"] = {"kernel": "pack_rows", "launch": pk.name, "bound": "hbm",
                                   "achieved": round(kp["GB/s"], 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(kp["frac_hbm"], 4),
                                   "traffic": measured_traffic("pack_rows", args.workload)}
    if not args.eager:
        result["ms_per_step_k_graph"] = round(ms_k_graph, 5)
    if not args.no_ceilings:
        from w8a8_int8_linear_amd import probe

        mf = probe.mfma_i8(dev)
        cp = probe.copy_gbps(dev)
        sw = probe.copy_sweep(dev)
        rd = probe.read_sweep(dev)
        result["ceilings"] = {
            "copy_GBps": cp["GBps"],
            "copy_by_grid": cp["by_grid_per_cu"],
            "torch_copy_GBps": cp["torch_copy_GBps"],
            "copy_fit": sw,
            "read_fit": rd,
            "mfma_i8_TOPS": mf["TOPS"],
            "mfma_i8_frac_of_peak": round(mf["TOPS"] / PEAK_I8_TOPS, 4),
            "sclk_GHz_mfma_loop": mf["sclk_GHz"],
            "sclk_GHz_range": [mf["sclk_GHz_min"], mf["sclk_GHz_max"]],
            "note": "streaming copy of 1 GiB (read + write bytes / s, best of three grid sizes); copy_fit and "
                    "read_fit: time = t0 + bytes / GBps fitted over graph-replayed copies and reads of 4-256 MiB; "
                    "MFMA-only "
                    "v_mfma_i32_16x16x64_i8 loop, one workgroup "
                    "per CU, two waves per SIMD, random normal codes; shader clock per CU from s_memtime against "
                    "the 100 MHz s_memrealtime",
        }
        if roof["bound"] == "mfma":
            roof["frac_of_measured_mfma"] = round(roof["achieved"] / mf["TOPS"], 4)
        else:
            roof["frac_of_copy"] = round(roof["achieved"] / result["ceilings"]["copy_GBps"], 4)
        def copy_floor_frac(op):
            # the op's measured time against a streaming copy of its bytes
            # (fixed cost plus bytes at the fitted bandwidth)
            best_us = sw["t0_us"] + op.bytes() / (sw["GBps"] * 1e3)
            return round(best_us / kernels[op.name]["us"], 4)

        if "pack_roofline" in result:
            result["pack_roofline"]["frac_of_copy"] = round(result["pack_roofline"]["achieved"] /
                                                            result["ceilings"]["copy_GBps"], 4)
            pk_op = [op for op in ops if op.name == result["pack_roofline"]["launch"]][0]
            result["pack_roofline"]["frac_of_sized_copy"] = copy_floor_frac(pk_op)
        if roof["bound"] == "hbm":
            roof["frac_of_sized_copy"] = copy_floor_frac(dom)
            # weight streaming is nearly all reads: its floor is a read of
            # its bytes
            roof["frac_of_sized_read"] = round((rd["t0_us"] + dom.bytes() / (rd["GBps"] * 1e3)) /
                                               kernels[dom.name]["us"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
