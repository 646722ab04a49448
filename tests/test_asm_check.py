"""The static wait-state check of the inline-asm MFMAs (bf16 and fp8 softmax, merged dK/dV backward): the
checker flags planted hazards in small assembly listings, and the kernels as compiled are clean."""
import shutil

import pytest

from video_diffusion_hybrid_sparse_amd import asm_check

HEAD = "_ZN3vdn17softmax_sw_kernelILi128EEEvNS_11SoftmaxArgsE:\n"


def listing(*lines):
    return HEAD + "".join("\t" + l + "\n" for l in lines) + "\ts_endpgm\n"


def test_valu_write_then_mfma_read_flagged():
    asm = listing("v_mov_b32_e32 v2, v9", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]")
    assert len(asm_check.check_asm(asm)) == 1


def test_two_wait_states_clear_it():
    asm = listing("v_mov_b32_e32 v2, v9", "s_nop 1", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]")
    assert asm_check.check_asm(asm) == []


def test_mfma_result_read_by_valu_flagged_until_fenced():
    mf = "v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], a[4:7], v[16:31]"
    assert asm_check.check_asm(listing(mf, "s_nop 7", "v_exp_f32_e32 v40, v20"))
    assert asm_check.check_asm(listing(mf, "s_nop 7", "s_nop 3", "v_exp_f32_e32 v40, v20")) == []


def test_fp8_mfma_result_needs_twenty_wait_states():
    """The 16-pass 32x32x64 fp8 MFMA: the 12 wait states that clear a bf16 result are not enough."""
    mf = "v_mfma_f32_32x32x64_f8f6f4 v[16:31], v[0:7], a[0:7], v[16:31]"
    assert asm_check.check_asm(listing(mf, "s_nop 7", "s_nop 3", "v_exp_f32_e32 v40, v20"))
    assert asm_check.check_asm(listing(mf, "s_nop 7", "s_nop 7", "s_nop 2", "v_exp_f32_e32 v40, v20"))
    assert asm_check.check_asm(listing(mf, "s_nop 7", "s_nop 7", "s_nop 3", "v_exp_f32_e32 v40, v20")) == []
    # an unrelated bf16 MFMA in between counts one wait state: the fp8 result still needs its 20
    bf = "v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], a[4:7], v[32:47]"
    assert asm_check.check_asm(listing(mf, bf, "s_nop 7", "s_nop 3", "v_exp_f32_e32 v40, v20"))
    assert asm_check.check_asm(listing(mf, "s_nop 7", bf, "s_nop 7", "s_nop 3", "v_exp_f32_e32 v40, v20")) == []


def test_execz_jump_counts_only_where_lanes_can_be_off():
    """s_cbranch_execz cannot jump while every lane is active (kernel entry, outside the
    compiler's saveexec regions); inside one it can."""
    body = ("\tv_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], a[4:7], v[16:31]\n\ts_cbranch_execz .LBB0_2\n"
            "\ts_nop 7\n\ts_nop 7\n.LBB0_2:\n\tv_mov_b32_e32 v20, 0\n\ts_endpgm\n")
    assert asm_check.check_asm(HEAD + body) == []
    divergent = HEAD + "\ts_and_saveexec_b64 s[0:1], vcc\n" + body
    assert len(asm_check.check_asm(divergent)) == 1
    restored = HEAD + "\ts_and_saveexec_b64 s[0:1], vcc\n\ts_or_b64 exec, exec, s[0:1]\n" + body
    assert asm_check.check_asm(restored) == []


def test_hazard_through_a_branch_flagged():
    asm = (HEAD + "\tv_mov_b32_e32 v5, 0\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 7\n"
           ".LBB0_2:\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]\n\ts_endpgm\n")
    assert len(asm_check.check_asm(asm)) == 1


def test_agpr_write_then_mfma_accumulate_flagged():
    asm = listing("v_accvgpr_write_b32 a3, v1", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]")
    assert len(asm_check.check_asm(asm)) == 1


def test_m0_write_right_before_lds_dma_flagged():
    """The LDS DMA copy reads its destination from M0: one wait state after the M0 write."""
    dma = "global_load_lds_dwordx4 v1, s[4:5]"
    assert len(asm_check.check_asm(listing("s_mov_b32 m0, s6", dma))) == 1
    assert asm_check.check_asm(listing("s_mov_b32 m0, s6", "s_nop 0", dma)) == []
    mf = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"
    assert asm_check.check_asm(listing("s_mov_b32 m0, s6", mf, dma)) == []


def test_valu_sgpr_write_then_memory_read_flagged():
    """v_readfirstlane into a copy's base address: five wait states before the copy."""
    rfl = "v_readfirstlane_b32 s5, v3"
    dma = "global_load_lds_dwordx4 v1, s[4:5]"
    assert len(asm_check.check_asm(listing(rfl, "s_mov_b32 m0, s6", "s_nop 0", dma))) == 1
    assert asm_check.check_asm(listing(rfl, "s_mov_b32 m0, s6", "s_nop 3", dma)) == []
    # an SGPR the copy does not read is no hazard
    assert asm_check.check_asm(listing("v_readfirstlane_b32 s9, v3", "s_mov_b32 m0, s6", "s_nop 0", dma)) == []


def test_compiler_use_of_m0_flagged_outside_inline_asm():
    plain = "\ts_mov_b32 m0, s4\n\tds_read_addtid_b32 v1\n"
    assert len(asm_check.check_m0(plain)) == 1
    in_asm = "\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\t;;#ASMEND\n\tv_mov_b32_e32 v1, v2\n"
    assert asm_check.check_m0(in_asm) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_kernels_as_compiled_are_clean():
    """The bf16 softmax and the merged dK/dV backward, compiled with the library's flags."""
    assert asm_check.check() == []
