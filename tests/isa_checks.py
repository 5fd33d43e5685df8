"""Static checks of the gfx950 assembly the kernels compile to.

The kernels issue their direct global->LDS copies from inline assembly, so
the compiler's hazard recognizer does not see those instructions.  These
checks read the assembly of our own build (hipcc --save-temps) and look for
hazards the inline assembly must cover itself.
"""

from __future__ import annotations

import os
import re
import subprocess
import tempfile


def _sregs(tok: str) -> set[int]:
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def valu_sgpr_vmem_hazards(asm: str, wait_states: int = 5) -> tuple[int, list[str]]:
    """VMEM instructions with an SGPR base (saddr) written by a VALU
    instruction fewer than `wait_states` wait states earlier in the same
    basic block.  Returns (number of saddr LDS-DMA sites, offending lines)."""
    sites = 0
    bad: list[str] = []
    hist: list[tuple[int, set[int]]] = []
    for raw in asm.split("\n"):
        s = raw.strip()
        if not s or s.startswith(";"):
            continue
        if re.match(r"^(\.LBB|_Z)\S*:", s):
            hist = []
            continue
        if s.startswith("."):
            continue
        op = s.split()[0]
        args = [a.strip() for a in s[len(op):].split(",")]
        if op.startswith("global_load_lds") and len(args) > 1 and args[1].startswith("s["):
            sites += 1
            need = _sregs(args[1])
            ws = 0
            for w, written in reversed(hist):
                if written & need:
                    if ws < wait_states:
                        bad.append(s)
                    break
                ws += w
                if ws >= wait_states:
                    break
        w = 1
        m = re.match(r"s_nop\s+(\d+)", s)
        if m:
            w = int(m.group(1)) + 1
        written = _sregs(args[0]) if (op.startswith("v_") and args) else set()
        hist.append((w, written))
    return sites, bad


def device_assembly(src: str, flags: list[str]) -> str:
    """Compile one HIP source for gfx950 and return its device assembly."""
    from exact_attention_51_amd import build

    with tempfile.TemporaryDirectory() as tmp:
        cmd = [build.hipcc(), *build.COMMON_FLAGS, *flags, "-c", src, "--save-temps", "-o", os.path.join(tmp, "x.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        (asm_file,) = [f for f in os.listdir(tmp) if f.endswith("gfx950.s")]
        return open(os.path.join(tmp, asm_file)).read()
