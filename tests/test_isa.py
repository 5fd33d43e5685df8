"""Build-level checks on the generated gfx950 code (no GPU needed)."""

import os

import pytest

from exact_attention_51_amd import build
from tests.isa_checks import device_assembly, valu_sgpr_vmem_hazards

KERNEL_SOURCES = [s for s in build.sources() if os.path.basename(s) not in build.HOST_ONLY_SOURCES]


@pytest.mark.slow
@pytest.mark.parametrize("src", KERNEL_SOURCES, ids=os.path.basename)
def test_direct_lds_copies_cover_valu_sgpr_hazard(src):
    """Every direct global->LDS copy with an SGPR base sits at least 5 wait
    states after a VALU write of that SGPR (v_readfirstlane) when that write
    is the most recent one.  With fewer, the copy can read a stale base
    address."""
    asm = device_assembly(src, build.source_flags(os.path.basename(src)))
    sites, bad = valu_sgpr_vmem_hazards(asm)
    assert not bad, f"{len(bad)} of {sites} copies too close to a VALU write of their base: {bad[:3]}"


def test_hazard_scanner_flags_a_planted_hazard():
    planted = """
_Zkernel:
    v_readfirstlane_b32 s82, v208
    v_readfirstlane_b32 s83, v207
    s_nop 0
    global_load_lds_dwordx4 v145, s[82:83]
    v_readfirstlane_b32 s4, v1
    s_nop 4
    global_load_lds_dwordx4 v145, s[4:5]
"""
    sites, bad = valu_sgpr_vmem_hazards(planted)
    assert sites == 2 and len(bad) == 1 and "s[82:83]" in bad[0]


def test_hazard_scanner_follows_the_most_recent_writer():
    """A scalar write after the VALU write supersedes it (no hazard); a VALU
    write after a scalar one is the one that counts."""
    code = """
_Zkernel:
    v_readfirstlane_b32 s28, v144
    s_add_u32 s28, s17, s28
    s_addc_u32 s29, s7, 0
    s_nop 0
    global_load_lds_dwordx4 v131, s[28:29]
    s_add_u32 s30, s17, s28
    v_readfirstlane_b32 s31, v1
    s_cmp_lt_i32 s31, s22
    global_load_lds_dwordx4 v131, s[30:31]
"""
    sites, bad = valu_sgpr_vmem_hazards(code)
    assert sites == 2 and bad == ["global_load_lds_dwordx4 v131, s[30:31]"]
