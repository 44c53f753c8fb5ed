"""The wait-state check the build runs over the device assembly of the inline-asm
global -> LDS copies (CDNA rule: 5 wait states between a VALU write of an SGPR and a
VMEM read of it; 1 between an SALU write of M0 and a load to LDS)."""
from mixture_experts_layer_03_amd import isa_check

FN = "_ZN3moe1kEv:\n"


def test_valu_written_base_read_at_once_is_flagged():
    # a spilled base restored with v_readlane and read by the copy right away
    asm = FN + """
	v_readlane_b32 s2, v109, 26
	s_mov_b32 m0, s2
	v_readlane_b32 s2, v109, 27
	v_readlane_b32 s3, v109, 28
	;;#ASMSTART
	global_load_lds_dwordx4 v42, s[2:3]
	;;#ASMEND
"""
    bad = isa_check.check(asm)
    assert bad and "v_readlane_b32 s3" in bad[0]


def test_salu_copy_of_the_base_passes():
    asm = FN + """
	v_readlane_b32 s2, v109, 27
	v_readlane_b32 s3, v109, 28
	s_mov_b32 m0, s4
	;;#ASMSTART
	s_mov_b64 s[6:7], s[2:3]
	global_load_lds_dwordx4 v42, s[6:7]
	;;#ASMEND
"""
    assert isa_check.check(asm) == []


def test_m0_write_right_before_a_copy_is_flagged():
    asm = FN + """
	s_mov_b32 m0, s4
	global_load_lds_dword v[38:39], off
"""
    assert any("M0" in b for b in isa_check.check(asm))
    ok = FN + """
	s_mov_b32 m0, s4
	s_nop 0
	global_load_lds_dword v[38:39], off
"""
    assert isa_check.check(ok) == []


def test_enough_wait_states_pass_and_labels_reset():
    asm = FN + """
	v_readfirstlane_b32 s8, v1
	v_readfirstlane_b32 s9, v2
	s_nop 4
	s_mov_b32 m0, s4
	s_nop 0
	global_load_lds_dwordx4 v1, s[8:9]
"""
    assert isa_check.check(asm) == []
    short = asm.replace("s_nop 4", "s_nop 1")
    assert isa_check.check(short)
