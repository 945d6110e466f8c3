"""Static checks of the generated gfx950 assembly: no matrix-core (MFMA)
instruction may be reachable with an empty EXEC mask, and no kernel may use
scratch memory (a register spill costs a memory round trip per use in the
hot loops; every kernel here is sized to fit its registers).

MFMA instructions do not honour the EXEC mask, so a divergent `if` around one
(which the compiler lowers to s_and_saveexec ... s_or_b64 exec without a
branch when the region is short) still executes it, on whatever the
operand registers hold.  Every MFMA-guarding condition in the kernels must
therefore be provably wave-uniform (a scalar branch), or at least skipped
by s_cbranch_execz when no lane is active.  This tool compiles the HIP
sources to assembly and reports any MFMA that follows an EXEC save without
such a skip.

Usage: python -m ulysses_sequence_parallelism_head_amd.isa_check
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from .build import COMMON, HIPCC, sources

_SAVE = re.compile(r"^\s*s_(and|or|andn2|orn2|xor)_saveexec_b64\s+(s\[\d+:\d+\])")
_RESTORE = re.compile(r"^\s*s_(or|mov|and)_b64\s+exec,\s*(?:exec,\s*)?(s\[\d+:\d+\])")
_FUNC = re.compile(r"^([A-Za-z_][\w.$]*):\s*(?:;.*)?$")
_LABEL = re.compile(r"^(\.L[\w$]+):")
_BRANCH = re.compile(r"^\s*(s_cbranch_\w+|s_branch)\s+(\.L[\w$]+)")
_MFMA = re.compile(r"^\s*v_mfma_")
_END = re.compile(r"^\s*(s_endpgm|s_setpc_b64)")


def scan(asm: str, max_steps: int = 20000):
    """Return [(function, line number, instruction)] of MFMAs that can run
    while EXEC may be empty: every path from an EXEC save is followed --
    through labels (fall-through), conditional branches on SCC or VCC (both
    ways), unconditional branches, and the taken side of s_cbranch_execz
    (EXEC is empty there) -- until EXEC is restored, the program ends, or
    s_cbranch_execz / s_cbranch_execnz leaves the empty-EXEC case behind.
    A walk that runs out of its step budget is reported too (inconclusive
    counts as a failure)."""
    lines = asm.splitlines()
    labels = {}
    func_of = []
    func = "?"
    for i, line in enumerate(lines):
        m = _FUNC.match(line)
        if m and not line.startswith("."):
            func = m.group(1)
        m = _LABEL.match(line)
        if m:
            labels[m.group(1)] = i
        func_of.append(func)

    bad = set()
    for start, line in enumerate(lines):
        if not _SAVE.match(line):
            continue
        stack, seen, steps = [start + 1], set(), 0
        while stack and steps < max_steps:
            i = stack.pop()
            while i < len(lines) and steps < max_steps:
                if i in seen:
                    break
                seen.add(i)
                steps += 1
                text = lines[i].strip()
                if _FUNC.match(lines[i]) and not lines[i].startswith("."):
                    break                                   # next function
                if _MFMA.match(lines[i]):
                    bad.add((func_of[i], i + 1, text))
                if _RESTORE.match(lines[i]) or _END.match(lines[i]):
                    break
                m = _BRANCH.match(lines[i])
                if m:
                    op, target = m.group(1), m.group(2)
                    tgt = labels.get(target)
                    if op == "s_branch":
                        if tgt is not None:
                            stack.append(tgt)
                        break
                    if op == "s_cbranch_execz":              # taken iff EXEC is empty
                        if tgt is not None:
                            stack.append(tgt)
                        break
                    if op == "s_cbranch_execnz":             # falls through iff EXEC is empty
                        i += 1
                        continue
                    if tgt is not None:                      # SCC / VCC: both ways
                        stack.append(tgt)
                i += 1
        if steps >= max_steps:
            bad.add((func_of[start], start + 1, "walk from this EXEC save exceeded its step budget"))
    return sorted(bad, key=lambda b: b[1])


_KERNEL = re.compile(r"^\s*\.amdhsa_kernel\s+(\S+)")
_PRIVATE = re.compile(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)")


def scratch_kernels(asm: str):
    """Return [(kernel, bytes per lane)] of kernels whose descriptor asks for
    a private (scratch) segment."""
    found = []
    kernel = None
    for line in asm.splitlines():
        m = _KERNEL.match(line)
        if m:
            kernel = m.group(1)
            continue
        m = _PRIVATE.match(line)
        if m and kernel is not None and int(m.group(1)) > 0:
            found.append((kernel, int(m.group(1))))
    return found


def check(verbose: bool = True):
    problems = []
    with tempfile.TemporaryDirectory() as tmp:
        for src in sources():
            out = os.path.join(tmp, os.path.basename(src) + ".s")
            cmd = [HIPCC, *COMMON, "--cuda-device-only", "-S", src, "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
            with open(out, encoding="utf-8") as f:
                asm = f.read()
            found = scan(asm)
            scratch = scratch_kernels(asm)
            n_mfma = sum(1 for l in asm.splitlines() if _MFMA.match(l))
            if verbose:
                print(f"{os.path.basename(src)}: {n_mfma} MFMA, {len(found)} reachable with an empty EXEC, "
                      f"{len(scratch)} kernels with scratch")
            problems += [(os.path.basename(src), *b) for b in found]
            problems += [(os.path.basename(src), k, 0, f"scratch: {n} bytes per lane") for k, n in scratch]
    return problems


if __name__ == "__main__":
    bad = check()
    for b in bad[:50]:
        print("  ", *b)
    sys.exit(1 if bad else 0)
