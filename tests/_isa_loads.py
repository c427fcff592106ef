"""Static check of gfx950 assembly: no instruction may touch a VGPR or AGPR that an LDS or global
load is still writing.

The kernels issue many of their LDS reads from inline assembly and wait for them with explicit
``s_waitcnt`` in a later statement, so that a ring of operand reads stays in flight across MFMAs.
The compiler sees such a read's destination as written when the asm statement ends; nothing but
the kernel's own waits keeps it from copying or reusing that register before the data lands (a
register allocator that copies the destination to another register class right after the read
would copy stale data).  This module reads the compiler's assembly of a kernel, follows its
control flow, counts the loads in flight per hardware counter (lgkmcnt: LDS and scalar memory,
in issue order for LDS; vmcnt: vector memory, in issue order) and reports every instruction that
reads or writes a register whose load the waits executed so far do not cover.

Model: a load's destination is pending from its issue until an ``s_waitcnt`` leaves at most N
newer operations of its counter in flight.  A later load of the same counter into a pending
register is not reported (loads of one counter return in order).  At a label the states of
every incoming edge are merged pessimistically (per counter, the longest queue, with the
destination sets of equally old entries united); loop back-edges are followed until the state at
each label stops changing.
"""
from __future__ import annotations

import re
from dataclasses import dataclass

_REG = re.compile(r"^([va])\[(\d+):(\d+)\]$|^([va])(\d+)$")
_LABEL = re.compile(r"^(\.?L\w+|\w+):")
_BRANCH = re.compile(r"^s_(cbranch_\w+|branch)\s+(\S+)")
# most operations a counter holds (gfx9: 4-bit lgkmcnt, 6-bit vmcnt); a wave issuing more waits for
# the oldest, so older entries are complete
_CAP = {"lgkm": 15, "vm": 63}


def _regs(tok: str) -> frozenset:
    tok = tok.strip()
    m = _REG.match(tok)
    if not m:
        return frozenset()
    if m.group(1):
        return frozenset(f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset([tok])


@dataclass(frozen=True)
class Ins:
    op: str
    dst: frozenset     # registers written (vector registers only)
    src: frozenset     # registers read
    text: str


def _kind(op: str):
    """(counter, returns data) of a memory instruction, or None."""
    if op.startswith("ds_"):
        ret = op.startswith(("ds_read", "ds_load", "ds_bpermute", "ds_permute", "ds_swizzle")) or "_rtn" in op
        return "lgkm", ret
    if op.startswith(("s_load", "s_buffer_load")):
        return "lgkm", False
    if op.startswith(("global_load", "buffer_load", "scratch_load")):
        return "vm", "_lds" not in op
    if op.startswith(("global_store", "buffer_store", "scratch_store")):
        return "vm", False
    if op.startswith(("global_atomic", "buffer_atomic")):
        return "vm", False
    if op.startswith("flat_"):
        return "flat", op.startswith("flat_load")
    return None


def parse(op_line: str) -> Ins | None:
    t = op_line.split(";")[0].strip()
    if not t or t.startswith(".") or _LABEL.match(t):
        return None
    op = t.split()[0]
    args = [a.strip() for a in t[len(op):].split(",")] if len(t) > len(op) else []
    k = _kind(op)
    # vector ALU and MFMA instructions, and loads that return data, name their destination first
    # (an SGPR or VCC destination yields no vector register)
    writes_first = bool(args) and (op.startswith("v_") or (k is not None and k[1]))
    dst = _regs(args[0]) if writes_first else frozenset()
    src = frozenset().union(*[_regs(a.split()[0]) for a in (args[1:] if writes_first else args) if a])
    return Ins(op, dst, src, t)


def _merge(a, b):
    """Pessimistic union of two states (dicts counter -> tuple of frozensets, oldest first)."""
    if a is None:
        return b
    out = {}
    for c in ("lgkm", "vm"):
        qa, qb = a[c], b[c]
        n = max(len(qa), len(qb))
        qa = (frozenset(),) * (n - len(qa)) + qa
        qb = (frozenset(),) * (n - len(qb)) + qb
        out[c] = tuple(x | y for x, y in zip(qa, qb))
    return out


def _step(state, ins: Ins, issues, where):
    if ins.op == "s_waitcnt":
        st = dict(state)
        for c in ("lgkm", "vm"):
            m = re.search(c + r"cnt\((\d+)\)", ins.text)
            if m:
                n = int(m.group(1))
                st[c] = st[c][-n:] if n else ()
        return st
    k = _kind(ins.op)
    pend = {c: frozenset().union(*state[c]) if state[c] else frozenset() for c in ("lgkm", "vm")}
    touched = ins.src | ins.dst
    for c in ("lgkm", "vm"):
        bad = touched & pend[c]
        if k is not None and k[1] and k[0] == c:
            bad = (ins.src & pend[c]) | (ins.dst & pend[c] - ins.dst)  # same-counter reload: in order
        if bad and not ins.op.startswith("s_"):
            issues.add((where, ins.text, tuple(sorted(bad))[:4]))
    st = dict(state)
    if k is not None:
        ctrs = ("lgkm", "vm") if k[0] == "flat" else (k[0],)
        for c in ctrs:
            st[c] = (st[c] + ((ins.dst if k[1] else frozenset()),))[-_CAP[c]:]
    return st


def check_function(lines) -> list:
    """Issues [(instruction index, text, registers)] of one function's assembly lines."""
    seq, labels = [], {}
    for l in lines:
        t = l.split(";")[0].strip()
        m = _LABEL.match(t)
        if m:
            labels[m.group(1)] = len(seq)
            continue
        ins = parse(l)
        if ins is not None:
            seq.append(ins)
    label_at = set(labels.values())
    empty = {"lgkm": (), "vm": ()}
    at_label = {}        # instruction index -> merged state on entry
    issues = set()
    work = [0]
    at_label[0] = empty
    visits = 0
    while work:
        start = work.pop()
        state = at_label[start]
        i = start
        while i < len(seq):
            visits += 1
            if visits > 200000:
                raise RuntimeError("state did not settle")
            ins = seq[i]
            state = _step(state, ins, issues, i)
            m = _BRANCH.match(ins.text)
            if m:
                tgt = labels.get(m.group(2))
                if tgt is not None:
                    new = _merge(at_label.get(tgt), state)
                    if new != at_label.get(tgt):
                        at_label[tgt] = new
                        work.append(tgt)
                if m.group(1) == "branch":
                    break
            if ins.op == "s_endpgm" or ins.op == "s_setpc_b64":
                break
            i += 1
            if i in at_label and i != start:
                merged = _merge(at_label[i], state)
                if merged == at_label[i]:
                    break  # this path adds nothing here
                at_label[i] = merged
                state = merged
            elif i in label_at:
                at_label[i] = state
    return sorted(issues)


def functions(asm_text: str) -> dict:
    """Kernel name -> its assembly lines (the text between its label and its .Lfunc_end)."""
    out, cur = {}, None
    for l in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+|\w+):\s*(;.*)?$", l)
        if m and not l.startswith("."):  # a top-level symbol starts a new entry
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is not None:
            if l.strip().startswith(".Lfunc_end"):
                cur = None
            else:
                out[cur].append(l)
    return out
