"""Static check of the gfx950 assembly that hipcc produced for the kernels.

Some LDS transpose reads are issued from inline asm, so the compiler does not
know that their results arrive later: it treats the destination registers as
written when the instruction issues.  The kernels wait for them with an asm
``s_waitcnt lgkmcnt(N)`` tied to the destination, but register allocation may
still insert a copy (or any other use) of those registers between the read and
the wait, which would consume stale data.  This module scans the device
assembly and proves, for every inline-asm LDS read, that no instruction touches
its destination registers before an ``s_waitcnt`` that covers it:

* LDS operations complete in issue order, so after ``s_waitcnt lgkmcnt(n)`` a
  read is complete when at least ``n`` LGKM-counted operations were issued after
  it (scalar memory loads return out of order, so with one of those issued
  after the read only ``lgkmcnt(0)`` counts);
* a read still pending at a branch is reported (the check does not follow
  control flow), so straight-line code between read and wait is required.

``check_file(path)`` returns a list of problems (empty when the file is safe);
the build runs it on every translation unit that uses the asm reads.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass, field

_VREG_RANGE = re.compile(r"\bv\[(\d+):(\d+)\]")
_VREG_ONE = re.compile(r"\bv(\d+)\b")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_BRANCH_PREFIXES = ("s_branch", "s_cbranch", "s_setpc", "s_swappc", "s_endpgm")


def _vregs(text: str) -> set[int]:
    regs: set[int] = set()
    for a, b in _VREG_RANGE.findall(text):
        regs.update(range(int(a), int(b) + 1))
    for a in _VREG_ONE.findall(_VREG_RANGE.sub(" ", text)):
        regs.add(int(a))
    return regs


def _lgkm_op(mnem: str) -> str | None:
    """'lds' for in-order LGKM operations, 'smem' for out-of-order ones."""
    if mnem.startswith("ds_") or mnem.startswith("flat_"):
        return "lds"
    if mnem.startswith(("s_load", "s_buffer_load", "s_scratch_load", "s_memtime",
                        "s_memrealtime", "s_sendmsg", "s_get_barrier_state")):
        return "smem"
    return None


@dataclass
class _Pending:
    regs: set[int]
    line: int
    after: int = 0          # LGKM operations issued after this read
    smem_after: bool = False


@dataclass
class Report:
    reads: int = 0
    problems: list[str] = field(default_factory=list)


def check_text(text: str, name: str = "<asm>") -> Report:
    rep = Report()
    pending: list[_Pending] = []
    in_asm = False
    func = "?"
    for ln, raw in enumerate(text.splitlines(), 1):
        stripped = raw.strip()
        if stripped.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if stripped.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = raw.split(";", 1)[0].rstrip()
        if not code.strip():
            continue
        if not code[0].isspace():          # label or directive at column 0
            if code.endswith(":") and not code.startswith("."):
                func = code[:-1]
            continue
        body = code.strip()
        if body.startswith("."):           # directive
            continue
        mnem, _, ops = body.partition(" ")
        if mnem == "s_waitcnt":
            m = _LGKM.search(ops)
            if m:
                n = int(m.group(1))
                pending = [p for p in pending
                           if not (p.after >= n and (n == 0 or not p.smem_after))]
            continue
        used = _vregs(ops)
        for p in pending:
            if p.regs & used:
                rep.problems.append(
                    f"{name}:{ln}: {func}: '{body}' uses v{sorted(p.regs)} of the LDS read "
                    f"at line {p.line} before its wait")
        if mnem.startswith(_BRANCH_PREFIXES) and pending:
            rep.problems.append(
                f"{name}:{ln}: {func}: branch with {len(pending)} asm LDS read(s) pending "
                f"(first at line {pending[0].line})")
            pending = []
        kind = _lgkm_op(mnem)
        if kind:
            for p in pending:
                p.after += 1
                p.smem_after |= kind == "smem"
        if in_asm and mnem.startswith("ds_read"):
            dst = ops.split(",", 1)[0]
            pending.append(_Pending(regs=_vregs(dst), line=ln))
            rep.reads += 1
    if pending:
        rep.problems.append(f"{name}: {len(pending)} asm LDS read(s) pending at end of file")
    return rep


def check_file(path: str) -> Report:
    with open(path) as f:
        return check_text(f.read(), path)


if __name__ == "__main__":
    bad = 0
    for path in sys.argv[1:]:
        r = check_file(path)
        print(f"{path}: {r.reads} asm LDS reads, {len(r.problems)} problem(s)")
        for p in r.problems[:20]:
            print("  " + p)
        bad += len(r.problems)
    sys.exit(1 if bad else 0)
