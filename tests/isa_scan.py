"""Scan of gfx950 assembly for wait states that inline-asm buffer instructions must supply
themselves (the compiler's hazard pass does not look inside an asm statement):

* a buffer/global instruction that reads an SGPR needs 5 wait states after a VALU
  instruction that wrote the SGPR (v_readfirstlane, v_readlane, v_cmp with an SGPR result,
  carry-out forms);
* a copy into LDS (buffer_load ... lds) needs 1 wait state after an SALU write of m0.

Wait states are counted as issued instructions (s_nop N counts N + 1). The scan is linear
within a function, so a hazard across a branch into a block is also reported.
"""

from __future__ import annotations

import re

_VMEM = ("buffer_", "global_", "flat_", "scratch_")


def _sgprs(tok: str) -> set[int]:
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line: str) -> list[str]:
    parts = line.split(None, 1)
    return [t.strip().split()[0] for t in parts[1].split(",") if t.strip()] if len(parts) > 1 else []


def _valu_sgpr_defs(op: str, ops: list[str]) -> set[int]:
    if not op.startswith("v_") or not ops:
        return set()
    defs = set()
    if op.startswith(("v_readfirstlane", "v_readlane", "v_cmp")):
        defs |= _sgprs(ops[0])
    if len(ops) > 1 and re.match(r"v_(add|sub|subrev|addc|subb|subbrev)_co_u32|v_mad_[ui]64_[ui]32|v_div_scale", op):
        defs |= _sgprs(ops[1])
    return defs


def scan(asm_text: str) -> list[str]:
    """Hazards at inline-asm buffer instructions, one line of text each."""
    found = []
    for func in re.split(r"\n(?=_Z\S*:)", asm_text):
        name = func.split(":", 1)[0]
        if not name.startswith("_Z"):
            continue
        ws = 0              # wait states issued so far
        valu_defs = []      # (wait-state count after the VALU instruction, SGPRs it wrote)
        m0_def = None
        in_asm = False
        for raw in func.split("\n"):
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not line or line.startswith((";", ".", "//")) or line.endswith(":"):
                continue
            op = line.split()[0]
            ops = _operands(line)
            if in_asm and op.startswith(_VMEM):
                used = set().union(*(_sgprs(t) for t in ops)) if ops else set()
                for at, regs in valu_defs:
                    if ws - at < 5 and used & regs:
                        found.append(f"{name}: '{line}' reads s{sorted(used & regs)} {ws - at} wait states "
                                     f"after a VALU write")
                if " lds" in line and m0_def is not None and ws - m0_def < 1:
                    found.append(f"{name}: '{line}' follows an m0 write with no wait state")
            defs = _valu_sgpr_defs(op, ops)
            if op.startswith("s_") and ops and ops[0] == "m0":
                m0_def = ws + 1
            ws += int(ops[0]) + 1 if op == "s_nop" and ops else 1
            if defs:
                valu_defs.append((ws, defs))
            valu_defs = [d for d in valu_defs if ws - d[0] < 8]
    return found
