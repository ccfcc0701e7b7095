"""Static check of the gfx950 assembly that hipcc produced for the kernels.

Some LDS reads are issued from inline asm, so the compiler does not know that
their results arrive later: it treats the destination registers as written
when the instruction issues.  The kernels wait for them with an asm
``s_waitcnt lgkmcnt(N)`` tied to the destination, but register allocation may
still insert a copy (or any other use) of those registers between the read and
the wait, which would consume stale data.  This module scans the device
assembly and proves, for every inline-asm LDS read, that on every control-flow
path no instruction touches its destination registers before an
``s_waitcnt`` that covers it:

* LDS operations complete in issue order, so after ``s_waitcnt lgkmcnt(n)`` a
  read is complete when at least ``n`` LDS operations were issued after it on
  the path: were it still pending, so would be every LDS operation after it,
  and the counter would exceed ``n``.  Scalar memory loads (and other
  LGKM-counted operations that return out of order) do not count towards
  ``n``; while pending they only raise the counter, so they never let such a
  wait pass early;
* each function is split into basic blocks at labels and branches, and the
  set of pending reads is propagated along every edge to a fixed point; where
  paths join, a read pending on any incoming path is pending, with the fewest
  LGKM operations seen after it on any of them (so the check is conservative).

``check_file(path)`` returns a report whose ``problems`` list is empty when the
file is safe; the build runs it on every translation unit that uses the asm
reads.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass, field

_VREG_RANGE = re.compile(r"\bv\[(\d+):(\d+)\]")
_VREG_ONE = re.compile(r"\bv(\d+)\b")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_LABEL = re.compile(r"^([.\w$]+):")
_COND_BRANCH = ("s_cbranch",)
_UNCOND_BRANCH = ("s_branch",)
_END = ("s_endpgm", "s_setpc", "s_trap")


def _vregs(text: str) -> set[int]:
    regs: set[int] = set()
    for a, b in _VREG_RANGE.findall(text):
        regs.update(range(int(a), int(b) + 1))
    for a in _VREG_ONE.findall(_VREG_RANGE.sub(" ", text)):
        regs.add(int(a))
    return regs


def _lgkm_op(mnem: str) -> str | None:
    """'lds' for LGKM operations that complete in order with the LDS reads
    (only these count towards a partial wait); None otherwise."""
    if mnem.startswith("ds_"):
        return "lds"
    return None


@dataclass
class _Inst:
    line: int
    text: str
    mnem: str
    ops: str
    in_asm: bool


@dataclass
class _Block:
    label: str | None
    insts: list[_Inst] = field(default_factory=list)
    succs: list[int] = field(default_factory=list)


@dataclass
class Report:
    reads: int = 0
    problems: list[str] = field(default_factory=list)


# pending state: read line -> [dest regs, LDS operations issued after it]
_State = dict


def _functions(lines):
    """Yield (name, [_Inst or label str]) for every function body in the file."""
    func, body, in_asm = None, [], False
    for ln, raw in enumerate(lines, 1):
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
        if not code[0].isspace():
            m = _LABEL.match(code)
            if m:
                name = m.group(1)
                if not name.startswith("."):          # a new function
                    if func is not None:
                        yield func, body
                    func, body = name, []
                elif func is not None:
                    body.append(name)                  # a basic-block label
            elif code.startswith(".end") or code.startswith(".size"):
                pass
            continue
        text = code.strip()
        if text.startswith(".") or func is None:
            continue
        mnem, _, ops = text.partition(" ")
        body.append(_Inst(ln, text, mnem, ops.strip(), in_asm))
    if func is not None:
        yield func, body


def _blocks(body) -> list[_Block]:
    blocks: list[_Block] = [_Block(None)]
    for item in body:
        if isinstance(item, str):
            if blocks[-1].insts or blocks[-1].label is not None:
                blocks.append(_Block(item))
            else:
                blocks[-1].label = item
            continue
        blocks[-1].insts.append(item)
        if item.mnem.startswith(_COND_BRANCH + _UNCOND_BRANCH + _END):
            blocks.append(_Block(None))
    index = {b.label: i for i, b in enumerate(blocks) if b.label is not None}
    for i, b in enumerate(blocks):
        last = b.insts[-1] if b.insts else None
        if last is not None and last.mnem.startswith(_END):
            continue
        if last is not None and last.mnem.startswith(_COND_BRANCH + _UNCOND_BRANCH):
            target = last.ops.split(",")[0].strip()
            if target in index:
                b.succs.append(index[target])
            if last.mnem.startswith(_UNCOND_BRANCH):
                continue
        if i + 1 < len(blocks):
            b.succs.append(i + 1)
    return blocks


def _transfer(block: _Block, state: _State, func: str, name: str, rep: Report | None):
    st = {k: list(v) for k, v in state.items()}
    for ins in block.insts:
        if ins.mnem == "s_waitcnt":
            m = _LGKM.search(ins.ops)
            if m:
                n = int(m.group(1))
                st = {k: v for k, v in st.items() if not v[1] >= n}
            continue
        # An LDS read's own destination may overlap a pending LDS read: LDS
        # returns in order, so the later value lands last.  Any other write
        # to (or read of) such a register is a hazard.
        used = (_vregs(ins.ops.split(",", 1)[1]) if ins.mnem.startswith("ds_read") and "," in ins.ops
                else _vregs(ins.ops))
        if rep is not None:
            for line, (regs, _) in st.items():
                if regs & used:
                    rep.problems.append(
                        f"{name}:{ins.line}: {func}: '{ins.text}' uses v{sorted(regs)} of the LDS "
                        f"read at line {line} before its wait")
        if _lgkm_op(ins.mnem):
            for v in st.values():
                v[1] += 1
        if ins.in_asm and ins.mnem.startswith("ds_read"):
            st[ins.line] = [_vregs(ins.ops.split(",", 1)[0]), 0]
    return st


def _join(a: _State, b: _State) -> _State:
    out = {k: list(v) for k, v in a.items()}
    for k, v in b.items():
        if k in out:
            out[k][1] = min(out[k][1], v[1])
        else:
            out[k] = list(v)
    return out


def check_text(text: str, name: str = "<asm>") -> Report:
    rep = Report()
    for func, body in _functions(text.splitlines()):
        rep.reads += sum(1 for i in body if isinstance(i, _Inst) and i.in_asm
                         and i.mnem.startswith("ds_read"))
        blocks = _blocks(body)
        ins_state: list[_State | None] = [None] * len(blocks)
        ins_state[0] = {}
        work = [0]
        while work:
            i = work.pop()
            out = _transfer(blocks[i], ins_state[i], func, name, None)
            for j in blocks[i].succs:
                new = out if ins_state[j] is None else _join(ins_state[j], out)
                if ins_state[j] is None or new != ins_state[j]:
                    ins_state[j] = new
                    work.append(j)
        for i, b in enumerate(blocks):
            if ins_state[i] is not None:
                _transfer(b, ins_state[i], func, name, rep)
    # one message per offending instruction
    rep.problems = sorted(set(rep.problems))
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
