"""Scan compiled gfx950 kernels for hazards around inline-asm memory instructions.

The compiler inserts the wait states that hardware hazards need before the
instructions it generates, but not before memory instructions written in
inline asm.  Two gfx9-family rules apply to the LDS DMAs issued that way:

* an LDS DMA reads M0, which needs 1 wait state after an SALU write of M0;
* a vector memory instruction reading an SGPR (a buffer descriptor, an
  SGPR offset) needs 5 wait states after a VALU write of that SGPR
  (v_readfirstlane, v_readlane, a VALU compare or carry into an SGPR).

The scan walks backwards from each memory instruction inside an inline-asm
block along every path that can reach it (s_nop N counts N+1 wait states,
any other instruction 1): at a label it follows both the fall-through from
the instruction above (unless that is an unconditional branch or the end of
the program) and every branch that targets the label, loop back-edges
included, until each path has gathered five wait states.  Run by build();
a finding fails the build.
"""
from __future__ import annotations

import re
import sys
from collections import defaultdict
from typing import List

_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")
_VMEM = ("buffer_", "global_", "scratch_", "flat_")
_BRANCH = re.compile(r"^s_(?:c)?branch(?:_\w+)?\s+(\S+)")
_NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc_b64")


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


def _is_label(t: str) -> bool:
    return t.endswith(":") and " " not in t


def _skip(t: str) -> bool:
    return not t or (t.startswith(".") and not _is_label(t)) or t.startswith(";")


def scan(asm: str) -> List[str]:
    lines = [l.split(";")[0].strip() if not l.strip().startswith(";;#ASM") else l.strip()
             for l in asm.splitlines()]
    branches_to = defaultdict(list)      # label -> line indices of the branches that target it
    for k, t in enumerate(lines):
        m = _BRANCH.match(t)
        if m:
            branches_to[m.group(1)].append(k)

    def previous(j):
        """Index of the nearest instruction or label above line j, or -1."""
        j -= 1
        while j >= 0 and _skip(lines[j]):
            j -= 1
        return j

    findings = []
    seen_findings = set()
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
        stack = [(previous(i), 0)]
        visited = set()
        while stack:
            j, ws = stack.pop()
            while j >= 0 and ws < 5:
                if (j, ws) in visited:
                    break
                visited.add((j, ws))
                t = lines[j]
                if _is_label(t):
                    for b in branches_to.get(t[:-1], ()):
                        stack.append((b, ws))
                    above = previous(j)
                    if above >= 0 and _split(lines[above])[0] in _NO_FALLTHROUGH:
                        break
                    j = above
                    continue
                top, tops = _split(t)
                if top == "s_nop":
                    ws += int(tops.split()[0], 0) + 1
                    j = previous(j)
                    continue
                dst = tops.split(",")[0].strip()
                msg = None
                if lds_dma and ws < 1 and dst == "m0":
                    msg = "line %d: LDS DMA %r reads M0 right after %r (line %d)" % (i + 1, line, t, j + 1)
                elif top.startswith("v_") and (_sregs(dst) & reads):
                    msg = ("line %d: %r reads an SGPR written by %r (line %d) %d wait states earlier"
                           % (i + 1, line, t, j + 1, ws))
                if msg and msg not in seen_findings:
                    seen_findings.add(msg)
                    findings.append(msg)
                ws += 1
                j = previous(j)
    return findings


if __name__ == "__main__":
    found = scan(open(sys.argv[1]).read())
    print("\n".join(found) if found else "no hazards")
    sys.exit(1 if found else 0)
