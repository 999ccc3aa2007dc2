"""Soundness check of the decode kernel's inline-asm load ring, on its AMDGPU
assembly.

The E4M3 decode issues its K/V loads as inline `global_load_dwordx4` and
retires them with its own `s_waitcnt vmcnt(N)`.  The compiler does not see
those loads as memory operations, so nothing stops the register allocator
from reading (copying) or reusing a destination register while its load is
still in flight.  That would read stale data, or let the landing load
overwrite an unrelated value.  This module proves, for one kernel's
assembly, that no instruction touches a register of an in-flight ring load.

Model (dataflow over the kernel's basic blocks, to a fixed point):
  * state: for every register of an inline-asm load still in flight, the
    least number of vector-memory operations issued after that load on any
    path (fewer younger operations = more likely still pending);
  * any vector-memory operation (global_/buffer_/flat_/scratch_, loads and
    stores alike, all counted by vmcnt on gfx9-family chips) ages every
    pending register by one; an inline-asm load then adds its destination
    registers with age 0;
  * `s_waitcnt vmcnt(N)` retires every register whose load has at least N
    younger operations (vector-memory returns are counted in issue order);
  * any other instruction that names a pending register, as source or
    destination, is a violation;
  * at a join the states merge by union, keeping the smaller age.
Inline-asm blocks are recognised by the assembler comments the compiler
puts around them.
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

_VMEM = re.compile(r"^(global_|buffer_|flat_|scratch_)")
_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
_LABEL = re.compile(r"^(\.LBB[\w]+):")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.LBB[\w]+)")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
AGE_CAP = 64


@dataclass
class Instr:
    text: str
    in_asm: bool
    line: int


@dataclass
class Block:
    name: str
    instrs: list = field(default_factory=list)
    succ: list = field(default_factory=list)


def kernel_body(asm: str, symbol: str) -> list[str]:
    """Lines of one function's body: from its label to its s_endpgm."""
    lines = asm.splitlines()
    start = None
    for i, l in enumerate(lines):
        if l.split(";")[0].strip() == symbol + ":":
            start = i + 1
            break
    if start is None:
        raise KeyError(symbol)
    out = []
    for l in lines[start:]:
        out.append(l)
        if l.strip().startswith(".Lfunc_end"):
            break
    return out


def _regs(operands: str) -> set[int]:
    regs = set()
    for m in _VREG.finditer(operands):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


def build_cfg(body: list[str]) -> list[Block]:
    blocks = [Block("entry")]
    in_asm = False
    for n, raw in enumerate(body):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = _LABEL.match(s)
        if m:
            prev = blocks[-1]
            nb = Block(m.group(1))
            if not prev.instrs or not _ends_unconditionally(prev.instrs[-1].text):
                prev.succ.append(nb.name)
            blocks.append(nb)
            continue
        code = s.split(";")[0].strip()
        if not code or code.startswith("."):
            continue
        blocks[-1].instrs.append(Instr(code, in_asm, n))
        b = _BRANCH.match(code)
        if b:
            blocks[-1].succ.append(b.group(2))
            nb = Block(f"after_{n}")
            if not code.startswith("s_branch"):
                blocks[-1].succ.append(nb.name)
            blocks.append(nb)
        elif code.startswith("s_endpgm"):
            blocks.append(Block(f"after_{n}"))
    return [b for b in blocks if b.instrs or b.succ]


def _ends_unconditionally(text: str) -> bool:
    return text.startswith("s_branch") or text.startswith("s_endpgm")


def _step(state: dict[int, int], ins: Instr, violations: list[str]) -> dict[int, int]:
    parts = ins.text.split(None, 1)
    op = parts[0]
    operands = parts[1] if len(parts) > 1 else ""
    if op == "s_waitcnt":
        m = _VMCNT.search(operands)
        if m:
            n = int(m.group(1))
            state = {r: a for r, a in state.items() if a < n}
        return state
    regs = _regs(operands)
    touched = regs & state.keys()
    if touched:
        violations.append(f"line {ins.line}: '{ins.text}' touches in-flight ring registers "
                          f"{sorted(touched)}")
    if _VMEM.match(op):
        state = {r: min(a + 1, AGE_CAP) for r, a in state.items()}
        if ins.in_asm and "load" in op:
            dst = operands.split(",")[0]
            for r in _regs(dst):
                state[r] = 0
    return state


def _merge(a: dict[int, int] | None, b: dict[int, int]) -> dict[int, int]:
    if a is None:
        return dict(b)
    out = dict(a)
    for r, age in b.items():
        out[r] = min(out.get(r, age), age)
    return out


def check(body: list[str]) -> tuple[list[str], int]:
    """Returns (violations, number of inline-asm loads seen)."""
    blocks = build_cfg(body)
    index = {b.name: b for b in blocks}
    n_ring = sum(1 for b in blocks for i in b.instrs if i.in_asm and i.text.startswith("global_load"))
    entry_state: dict[str, dict[int, int] | None] = {b.name: None for b in blocks}
    entry_state[blocks[0].name] = {}
    work = [blocks[0].name]
    violations: list[str] = []
    seen = set()
    while work:
        name = work.pop()
        blk = index[name]
        st = dict(entry_state[name])
        local: list[str] = []
        for ins in blk.instrs:
            st = _step(st, ins, local)
        for v in local:
            if v not in seen:
                seen.add(v)
                violations.append(v)
        for s in blk.succ:
            if s not in index:
                continue
            merged = _merge(entry_state[s], st)
            if merged != entry_state[s]:
                entry_state[s] = merged
                work.append(s)
    return violations, n_ring
