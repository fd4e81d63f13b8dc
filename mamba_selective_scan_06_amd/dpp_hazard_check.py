"""Check generated gfx950 assembly for the VALU-write -> DPP-read hazard.

On the gfx9 family a VALU instruction that reads a VGPR through a DPP
modifier needs two wait states after the last VALU instruction that wrote
that VGPR.  The compiler inserts them for DPP it generates itself, but not
for DPP written in inline asm, where the NSPLIT readout places s_nop by hand.
This checker walks every DPP instruction of an assembly listing backwards
through its basic block and reports any VALU write of the DPP source with
fewer than two wait states in between.  A label inside the window (another
path could enter there) counts as a violation unless the window is already
covered.

    python -m mamba_selective_scan_06_amd.dpp_hazard_check FILE.s [...]
"""
from __future__ import annotations

import re
import sys

_REG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")


def _regs(operand: str) -> set[int]:
    out: set[int] = set()
    for m in _REG.finditer(operand):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _split(line: str):
    """(mnemonic, operands) of an instruction line, or None for non-instructions."""
    code = line.split(";", 1)[0].strip()
    if not code or code.startswith(".") or code.endswith(":"):
        return None
    parts = code.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def check_lines(lines: list[str], name: str = "<asm>") -> list[str]:
    """Problems found for the DPP instructions written in inline asm (between
    the compiler's ;;#ASMSTART and ;;#ASMEND markers); the compiler resolves
    the hazard itself for the DPP it generates."""
    problems = []
    in_asm = False
    for i, line in enumerate(lines):
        marker = line.strip()
        if marker.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if marker.startswith(";;#ASMEND"):
            in_asm = False
            continue
        ins = _split(line)
        if ins is None or not in_asm:
            continue
        mnem, ops = ins
        if not mnem.startswith("v_") or "_dpp" not in mnem or len(ops) < 2:
            continue
        src = _regs(ops[1].split()[0])  # the DPP-modified operand is src0
        waits = 0
        j = i - 1
        while j >= 0 and waits < 2:
            prev = lines[j].split(";", 1)[0].strip()
            if prev.endswith(":"):
                problems.append(f"{name}:{i + 1}: label within two wait states before `{line.strip()}`")
                break
            pins = _split(lines[j])
            if pins is not None:
                pm, pops = pins
                if pm.startswith("v_") and pops and _regs(pops[0]) & src:
                    problems.append(f"{name}:{i + 1}: `{line.strip()}` reads a VGPR written "
                                    f"{waits} wait state(s) earlier by `{lines[j].strip()}`")
                    break
                if pm == "s_nop":
                    waits += int(pops[0], 0) + 1 if pops else 1
                else:
                    waits += 1
            j -= 1
    return problems


def check_file(path: str) -> list[str]:
    with open(path) as f:
        return check_lines(f.read().split("\n"), path)


def main(argv: list[str]) -> int:
    bad = []
    for p in argv:
        bad += check_file(p)
    for b in bad:
        print(b)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
