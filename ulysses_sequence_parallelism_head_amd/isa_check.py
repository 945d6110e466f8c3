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
_MFMA = re.compile(r"^\s*v_mfma_")


def scan(asm: str):
    """Return [(function, line number, instruction)] of MFMAs reached straight
    after an EXEC save, i.e. before any branch, jump target or EXEC restore:
    such an MFMA runs even when the saved mask leaves no lane active."""
    bad = []
    func = "?"
    lines = asm.splitlines()
    for no, line in enumerate(lines, 1):
        m = _FUNC.match(line)
        if m and not line.startswith("."):
            func = m.group(1)
            continue
        if not _SAVE.match(line):
            continue
        for j in range(no, min(no + 400, len(lines))):
            nxt = lines[j].strip()
            if not nxt or nxt.startswith(";"):
                continue                      # comments, fall-through block markers
            if nxt.startswith(".LBB") or nxt.startswith("s_cbranch") or nxt.startswith("s_branch") \
                    or _RESTORE.match(lines[j]) or nxt.startswith("s_endpgm") or nxt.startswith("s_setpc"):
                break
            if _MFMA.match(lines[j]):
                bad.append((func, j + 1, nxt))
    return bad


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
