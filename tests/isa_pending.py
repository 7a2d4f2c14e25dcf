"""Scan of gfx950 assembly for accesses to the destination registers of inline-asm vector
loads before the wait that covers them.

A kernel may issue buffer/global loads into VGPRs from inline assembly and wait for them
itself (s_waitcnt vmcnt(N) waits until at most N vector-memory operations of the wave are
outstanding; they complete in issue order). The compiler does not know that such a register
is filled later: it may read it, copy it, spill it or give it to another value before the
data has arrived, any of which reads or overwrites the wrong value. This scan follows the
control-flow graph of each function and, at every instruction, knows for each asm load
that may still be in flight the fewest vector-memory operations issued after it on any path
(a load is covered by vmcnt(N) once N or more operations followed it on every path). Any
instruction that names a register of such a load, other than the load itself, is reported.
"""

from __future__ import annotations

import re

_VMEM = ("buffer_", "global_", "flat_", "scratch_")
_CAP = 64


def _vregs(tok: str) -> frozenset:
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _operands(text: str) -> list[str]:
    parts = text.split(None, 1)
    return [t.strip().split()[0] for t in parts[1].split(",") if t.strip()] if len(parts) > 1 else []


def _parse(body: str):
    insts, labels, in_asm = [], {}, False
    for raw in body.split("\n"):
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        line = line.split(";")[0].strip()
        if not line:
            continue
        m = re.match(r"^(\S+):$", line)
        if m:
            labels.setdefault(m.group(1), []).append(len(insts))
            continue
        if line.startswith("."):
            continue
        insts.append((line.split()[0], _operands(line), line, in_asm))
    return insts, labels


def scan_function(body: str) -> list[str]:
    insts, labels = _parse(body)
    n = len(insts)

    def target(tok: str, at: int) -> int:
        m = re.match(r"(\d+)([fb])$", tok)
        if m:   # assembler-local label inside an asm statement
            cands = labels.get(m.group(1), [])
            return min(c for c in cands if c > at) if m.group(2) == "f" else max(c for c in cands if c <= at)
        return labels[tok][0]

    def succs(i: int) -> list[int]:
        op, ops, _, _ = insts[i]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [target(ops[0], i)]
        if op.startswith("s_cbranch"):
            return [target(ops[0], i), i + 1]
        return [i + 1] if i + 1 < n else []

    state_in = {0: {}}
    work = [0]
    found = set()
    while work:
        i = work.pop()
        st = dict(state_in[i])
        op, ops, text, in_asm = insts[i]
        m = re.search(r"vmcnt\((\d+)\)", text) if op == "s_waitcnt" else None
        if m:
            k = int(m.group(1))
            st = {s: v for s, v in st.items() if v[1] < k}
        else:
            used = frozenset().union(*[_vregs(t) for t in ops]) if ops else frozenset()
            for s, (regs, _) in st.items():
                if s != i and regs & used:
                    found.add(f"'{text}' uses v{sorted(regs & used)} before the wait for '{insts[s][2]}'")
            if op.startswith(_VMEM):
                st = {s: (r, min(c + 1, _CAP)) for s, (r, c) in st.items()}
                if in_asm and op.startswith(("buffer_load", "global_load")) and not text.endswith(" lds"):
                    st[i] = (_vregs(ops[0]), 0)
        for j in succs(i):
            old = state_in.get(j)
            if old is None:
                state_in[j] = st
                work.append(j)
                continue
            merged, changed = dict(old), False
            for s, (r, c) in st.items():
                if s not in merged or c < merged[s][1]:
                    merged[s] = (r, c)
                    changed = True
            if changed:
                state_in[j] = merged
                work.append(j)
    return sorted(found)


def scan(asm_text: str) -> list[str]:
    """Problems in every function of a gfx950 assembly listing, one line of text each."""
    out = []
    for func in re.split(r"\n(?=_Z\S*:)", asm_text):
        name = func.split(":", 1)[0]
        if not name.startswith("_Z") or "\n" not in func:
            continue
        out += [f"{name}: {p}" for p in scan_function(func.split("\n", 1)[1])]
    return out
