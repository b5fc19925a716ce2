"""Audit of the device assembly for loads written in inline asm.

Some kernels issue global loads through inline asm and retire them later with
an explicit, counted ``s_waitcnt vmcnt`` (so that the compiler adds no wait of
its own and more loads stay in flight). The compiler takes such a load's
destination registers as written when the asm statement ends: if it copied,
read or reused one of them before the counted wait, the instruction would see
stale data, or the load would land on top of a later value (an address, say).
The kernels name the loaded registers in the asm statement of the wait, which
keeps them live until then, but the register allocator could still move them.

This audit reads the device assembly that the build writes next to the
objects and replays each function in program order: vector-memory operations
enter a queue in issue order, ``s_waitcnt vmcnt(N)`` retires them from the
front until at most N remain (loads return in order), and any instruction
other than a later load into the same registers that names a destination
register of an inline-asm load still in the queue is reported. Loads the
compiler wrote itself are counted in the queue but not checked: the compiler
places their waits. The replay follows the text order of the function, which
matches the kernels' structure here (asm loads and their waits in unrolled
straight-line code and loop bodies).
"""

import glob
import os
import re

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_VMEM_PREFIX = ("global_", "buffer_", "flat_", "scratch_")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            lo, hi = int(m.group(4)), int(m.group(5))
            out.update((m.group(3), r) for r in range(lo, hi + 1))
    return out


def _vmcnt(operands):
    """The vmcnt an s_waitcnt sets, or None if it leaves vmcnt alone."""
    ops = operands.strip()
    m = re.search(r"vmcnt\((0x[0-9a-fA-F]+|\d+)\)", ops)
    if m:
        return int(m.group(1), 0)
    if re.fullmatch(r"0x0*|0+", ops):  # the all-zero immediate waits for everything
        return 0
    return None


def audit_function(lines, name="?"):
    """Findings [(name, line index, instruction, registers)] for one function's lines."""
    queue = []  # per outstanding vector-memory op: destination registers (asm loads only)
    in_asm = False
    found = []
    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        text = raw.split(";")[0].strip()
        if not text or text.endswith(":") or text.startswith("."):
            continue
        op, _, operands = text.partition(" ")
        if op == "s_waitcnt":
            n = _vmcnt(operands)
            if n is not None:
                del queue[:max(len(queue) - n, 0)]
            continue
        is_vmem = op.startswith(_VMEM_PREFIX)
        is_load = is_vmem and "_load" in op and "lds" not in op and " lds" not in operands
        pending = set().union(*queue) if queue else set()
        if pending:
            touched = _regs(operands)
            if is_load:
                # a later load may overwrite the same registers (they return
                # in order); only its address operands are reads
                touched = _regs(operands.split(",", 1)[1] if "," in operands else "")
            hit = touched & pending
            if hit:
                found.append((name, i, text, sorted(hit)))
        if is_vmem:
            dest = _regs(operands.split(",")[0]) if (is_load and in_asm) else set()
            queue.append(dest)
    return found


def audit_file(path):
    """Findings over every function of one device assembly file."""
    lines = open(path).read().splitlines()
    found = []
    i = 0
    while i < len(lines):
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", lines[i])
        if m and not m.group(1).startswith("."):
            j = i + 1
            while j < len(lines) and not lines[j].strip().startswith(".Lfunc_end"):
                j += 1
            if j < len(lines):
                found += [(f"{os.path.basename(path)}:{fn}", i + 2 + k, t, r)
                          for fn, k, t, r in audit_function(lines[i + 1:j], m.group(1))]
                i = j
        i += 1
    return found


def device_assembly(build_dir):
    return sorted(glob.glob(os.path.join(build_dir, "*-hip-amdgcn-amd-amdhsa-*.s")))


def audit_dir(build_dir):
    found = []
    for path in device_assembly(build_dir):
        found += audit_file(path)
    return found
