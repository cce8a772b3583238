"""Static check of compiled gfx950 kernels: LDS-read register hazards.

The GEMM kernels issue their LDS fragment reads (ds_read_b128) as inline
assembly, so the compiler does not know that the destination registers are
written asynchronously, some cycles later, and that only an
``s_waitcnt lgkmcnt`` makes them safe to touch.  If register allocation or
scheduling places any other instruction on such a register before the wait,
a late LDS write can silently corrupt it -- for an address register, a
memory fault.

This module parses the assembly the compiler emits (``-S`` for the device),
builds each kernel's control-flow graph and computes, as a forward dataflow
with the union of all predecessor states at joins, the ordered list of
outstanding LDS operations and the VGPRs each will write.  ``s_waitcnt
lgkmcnt(N)`` retires all but the N most recent.  Any instruction that reads
or writes a VGPR still owed by an outstanding LDS read is reported.

Only LDS reads are tracked: scalar memory loads also count against lgkmcnt
and are modelled as slots that write no vector register, which keeps the
count conservative.
"""

from __future__ import annotations

import re
from dataclasses import dataclass, field

_VRANGE = re.compile(r"(?<![a-z_])v\[(\d+):(\d+)\]")
_VSINGLE = re.compile(r"(?<![a-z_\[])v(\d+)\b")
_LABEL = re.compile(r"^(\.LBB\w+):")
_FUNC = re.compile(r"\n(?=\S+:\s*; @)")


def _vregs(text: str) -> set[int]:
    regs: set[int] = set()
    for m in _VRANGE.finditer(text):
        regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in _VSINGLE.finditer(text):
        regs.add(int(m.group(1)))
    return regs


@dataclass
class KernelReport:
    name: str
    vgprs: int
    agprs: int
    scratch_bytes: int
    mfma: int
    hazards: list[tuple[str, list[int]]] = field(default_factory=list)


def _parse(body: str) -> tuple[list[str], dict[str, int]]:
    insts: list[str] = []
    labels: dict[str, int] = {}
    for raw in body.split("\n"):
        line = raw.strip()
        if not line or line.startswith(";"):
            continue
        m = _LABEL.match(line)
        if m:
            labels[m.group(1)] = len(insts)
            continue
        if line.startswith("."):
            continue
        insts.append(line.split(";")[0].strip())
    return insts, labels


def _successors(insts: list[str], labels: dict[str, int]) -> list[list[int]]:
    n = len(insts)
    succ: list[list[int]] = []
    for i, t in enumerate(insts):
        op = t.split()[0] if t else ""
        tgt = re.search(r"(\.LBB\w+)", t)
        nxt = [i + 1] if i + 1 < n else []
        if op == "s_branch":
            succ.append([labels[tgt.group(1)]])
        elif op.startswith("s_cbranch"):
            succ.append([labels[tgt.group(1)]] + nxt)
        elif op in ("s_endpgm", "s_setpc_b64"):
            succ.append([])
        else:
            succ.append(nxt)
    return succ


def _join(a, b):
    if a is None:
        return b
    if b is None:
        return a
    width = max(len(a), len(b))
    aa = (frozenset(),) * (width - len(a)) + a
    bb = (frozenset(),) * (width - len(b)) + b
    return tuple(x | y for x, y in zip(aa, bb))


def scan_kernel(name: str, body: str) -> KernelReport:
    insts, labels = _parse(body)
    succ = _successors(insts, labels)
    state: list = [None] * len(insts)
    if insts:
        state[0] = tuple()
    work = [0] if insts else []
    hazards: dict[int, tuple[str, list[int]]] = {}
    while work:
        i = work.pop()
        st = list(state[i])
        t = insts[i]
        op = t.split()[0] if t else ""
        owed = set().union(*st) if st else set()
        if op.startswith("ds_read") or op.startswith("ds_load"):
            m = re.match(r"\S+\s+(v\[\d+:\d+\]|v\d+)", t)
            dst = _vregs(m.group(1)) if m else set()
            touched = _vregs(t)
            if touched & owed:
                hazards[i] = (t, sorted(touched & owed))
            st.append(frozenset(dst))
        elif op.startswith("ds_") or op.startswith("s_load") or op.startswith("s_buffer_load"):
            if _vregs(t) & owed:
                hazards[i] = (t, sorted(_vregs(t) & owed))
            st.append(frozenset())
        elif op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                keep = int(m.group(1))
                st = st[len(st) - keep:] if 0 < keep < len(st) else ([] if keep == 0 else st)
        elif _vregs(t) & owed:
            hazards[i] = (t, sorted(_vregs(t) & owed))
        out = tuple(st[-16:])
        for j in succ[i]:
            new = _join(state[j], out)
            if new != state[j]:
                state[j] = new
                work.append(j)

    def meta(key: str) -> int:
        m = re.search(key + r":\s*(\d+)", body)
        return int(m.group(1)) if m else -1

    return KernelReport(name, meta("NumVgprs"), meta("NumAgprs"), meta("ScratchSize"),
                        sum(1 for t in insts if t.startswith("v_mfma")), list(hazards.values()))


def scan_asm(text: str) -> list[KernelReport]:
    reports = []
    for part in _FUNC.split(text):
        m = re.match(r"(\S+):\s*; @", part)
        if m:
            reports.append(scan_kernel(m.group(1), part))
    return reports
