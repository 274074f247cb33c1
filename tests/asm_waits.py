"""Checker for gfx950 assembly of kernels that issue loads through inline asm
and wait for them with explicit `s_waitcnt vmcnt(N)`.

The compiler does not know such loads are in flight, so it could read (or
reuse) a destination register before the load has landed.  Walking the
instructions in order, every vector-memory operation is counted (loads
return in issue order); `s_waitcnt vmcnt(N)` retires all but the last N.
Any other instruction that reads or writes a destination register of a load
still outstanding is a violation.
"""

from __future__ import annotations

import re

_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([va])(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _RANGE.finditer(text):
        out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
    for m in _SINGLE.finditer(_RANGE.sub(" ", text)):
        out.add(f"{m.group(1)}{m.group(2)}")
    return out


def check_kernel(lines) -> list:
    """Violations (instruction texts) in one kernel's instruction lines."""
    pending = []  # destination register sets (None: no register result), issue order
    bad = []
    for raw in lines:
        t = raw.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        op, _, args = t.partition(" ")
        if op == "s_waitcnt":
            vm = re.search(r"vmcnt\((\d+)\)", args)
            if vm:
                del pending[: max(0, len(pending) - int(vm.group(1)))]
            continue
        live = set().union(*[d for d in pending if d]) if pending else set()
        vmem = op.startswith(("global_", "buffer_", "flat_", "scratch_"))
        if vmem and "load" in op and "lds" not in op:
            parts = [p.strip() for p in args.split(",")]
            dst = _regs(parts[0])
            if _regs(args) & live:
                bad.append(t)
            pending.append(dst)
            continue
        if _regs(args) & live:
            bad.append(t)
        if vmem:
            pending.append(None)
    return bad


def check_assembly(text: str, kernel_pattern: str):
    """(number of kernels matched, list of (kernel, violation))."""
    src = text.splitlines()
    pat = re.compile(kernel_pattern)
    found, bad = 0, []
    i = 0
    while i < len(src):
        line = src[i]
        if re.match(r"^_Z\S+:", line) and pat.search(line):
            name = line.split(":")[0]
            j = i + 1
            while j < len(src) and "s_endpgm" not in src[j]:
                j += 1
            found += 1
            bad += [(name, v) for v in check_kernel(src[i + 1 : j + 1])]
            i = j
        i += 1
    return found, bad
