"""Scan compiled gfx950 kernels for hazards around inline-asm memory instructions.

The compiler inserts the wait states that hardware hazards need before the
instructions it generates, but not before memory instructions written in
inline asm.  Two gfx9-family rules apply to the LDS DMAs issued that way:

* an LDS DMA reads M0, which needs 1 wait state after an SALU write of M0;
* a vector memory instruction reading an SGPR (a buffer descriptor, an
  SGPR offset) needs 5 wait states after a VALU write of that SGPR
  (v_readfirstlane, v_readlane, a VALU compare or carry into an SGPR).

The scan walks backwards from each memory instruction inside an inline-asm
block through the instructions before it in program order (s_nop N counts
N+1 wait states, any other instruction 1).  Program order also covers the
fall-through into a block; a block entered by a branch from elsewhere is
covered because every SGPR the DMAs read is settled before the loop that
issues them.  Run by build(); a finding fails the build.
"""
from __future__ import annotations

import re
import sys
from typing import List

_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_VMEM = ("buffer_", "global_", "scratch_", "flat_")


def _sregs(text: str) -> set:
    out = set()
    for m in _SREG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split(line: str):
    parts = line.split(None, 1)
    return parts[0], (parts[1] if len(parts) > 1 else "")


def scan(asm: str) -> List[str]:
    lines = [l.split(";")[0].strip() if not l.strip().startswith(";;#ASM") else l.strip()
             for l in asm.splitlines()]
    findings = []
    in_asm = False
    for i, line in enumerate(lines):
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not in_asm or not line.startswith(_VMEM):
            continue
        op, ops = _split(line)
        reads = _sregs(ops)
        lds_dma = op.startswith("global_load_lds") or ops.rstrip().endswith(" lds")
        ws, j = 0, i - 1
        while j >= 0 and ws < 5:
            t = lines[j]
            j -= 1
            if not t or t.startswith(".") or t.startswith(";"):
                continue
            top, tops = _split(t)
            if top == "s_nop":
                ws += int(tops.split()[0], 0) + 1
                continue
            dst = tops.split(",")[0].strip()
            if lds_dma and ws < 1 and dst == "m0":
                findings.append("line %d: LDS DMA %r reads M0 right after %r" % (i + 1, line, t))
            if top.startswith("v_") and (_sregs(dst) & reads):
                findings.append("line %d: %r reads an SGPR written by %r %d wait states earlier"
                                % (i + 1, line, t, ws))
            ws += 1
    return findings


if __name__ == "__main__":
    found = scan(open(sys.argv[1]).read())
    print("\n".join(found) if found else "no hazards")
    sys.exit(1 if found else 0)
