"""Build-time hazard check of the inline-asm score MFMAs of the fused prefill (no GPU needed): the
checker flags a VALU write of an MFMA operand within two instructions of the MFMA, and the kernel's
generated code has none."""
import shutil

import pytest

from dual_chunk_attention_amd import build, hazards

CLEAN = """
	ds_read_b128 v[10:13], v1 offset:512
	v_add_u32_e32 v40, s2, v41
	s_waitcnt lgkmcnt(0)
	;;#ASMSTART
	v_mfma_f32_32x32x16_bf16 v[20:35], v[10:13], v[50:53], v[20:35]
	;;#ASMEND
"""


def test_checker_accepts_operands_from_lds_and_other_vgprs():
    bad, blocks = hazards.asm_mfma_violations(CLEAN)
    assert blocks == 1 and bad == []


@pytest.mark.parametrize("write", ["v_mov_b32_e32 v11, v3", "v_add_f32_e32 v52, v1, v2",
                                   "v_mov_b32_e32 v27, 0"])
def test_checker_flags_a_valu_write_of_an_operand(write):
    isa = CLEAN.replace("	s_waitcnt lgkmcnt(0)\n", f"	{write}\n")
    bad, blocks = hazards.asm_mfma_violations(isa)
    assert blocks == 1 and len(bad) == 1 and write in bad[0][1]


def test_checker_counts_two_instructions_back():
    isa = CLEAN.replace("	v_add_u32_e32 v40, s2, v41\n", "	v_mov_b32_e32 v12, v3\n")
    assert len(hazards.asm_mfma_violations(isa)[0]) == 1       # second instruction back
    isa = CLEAN.replace("	ds_read_b128 v[10:13], v1 offset:512\n", "	v_mov_b32_e32 v12, v3\n")
    assert hazards.asm_mfma_violations(isa)[0] == []            # third instruction back


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_fused_prefill_generated_code_has_no_asm_mfma_hazard():
    import os
    for f in build.HAZARD_CHECKED:
        assert hazards.check_source(os.path.join(build.CSRC, f), build.FLAGS) > 0
