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


# scalar instructions whose first operand is a source, not a destination
_SALU_NO_SDST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_setprio",
                 "s_sendmsg", "s_endpgm", "s_sleep", "s_trap", "s_icache", "s_dcache", "s_set", "s_ttrace",
                 "s_store", "s_buffer_store", "s_atomic", "s_scratch_store")


def _sgpr_writes(op: str, args: list[str]) -> tuple[set[int], bool]:
    """SGPRs an instruction writes through its first operand, and whether it
    is a VALU instruction (v_readfirstlane, v_cmp with an SGPR pair, ...)."""
    if not args:
        return set(), False
    if op.startswith("v_"):
        return _sregs(args[0]), True
    if op.startswith("s_") and not op.startswith(_SALU_NO_SDST):
        return _sregs(args[0]), False
    return set(), False


def valu_sgpr_vmem_hazards(asm: str, wait_states: int = 5) -> tuple[int, list[str]]:
    """VMEM instructions with an SGPR base (saddr) whose most recent writer,
    in the same basic block, is a VALU instruction fewer than `wait_states`
    wait states earlier (a later scalar write of the same SGPR supersedes
    it).  Returns (number of saddr LDS-DMA sites, offending lines)."""
    sites = 0
    bad: list[str] = []
    hist: list[tuple[int, set[int], bool]] = []
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
            need = set(_sregs(args[1]))
            ws = 0
            for w, written, valu in reversed(hist):
                hit = written & need
                if hit:
                    if valu and ws < wait_states:
                        bad.append(s)
                        break
                    need -= hit  # this writer is the most recent one for these SGPRs
                    if not need:
                        break
                ws += w
                if ws >= wait_states:  # older VALU writes are far enough back
                    break
        w = 1
        m = re.match(r"s_nop\s+(\d+)", s)
        if m:
            w = int(m.group(1)) + 1
        written, valu = _sgpr_writes(op, args)
        hist.append((w, written, valu))
    return sites, bad


def device_assembly(src: str, flags: list[str]) -> str:
    """Compile one HIP source for gfx950 and return its device assembly."""
    from exact_attention_51_amd import build

    with tempfile.TemporaryDirectory() as tmp:
        cmd = [build.hipcc(), *build.COMMON_FLAGS, *flags, "-c", src, "--save-temps", "-o", os.path.join(tmp, "x.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        (asm_file,) = [f for f in os.listdir(tmp) if f.endswith("gfx950.s")]
        return open(os.path.join(tmp, asm_file)).read()
