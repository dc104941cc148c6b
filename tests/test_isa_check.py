"""The build-time hazard check of accumulator accesses near inline-asm MFMAs
(gemm_epilogue_transformer_gemm1_amd/isa_check.py), on small hand-written
gfx950 assembly: straight-line code, across a conditional branch, across a
loop back-edge, and blocks that only a distant branch reaches."""
from gemm_epilogue_transformer_gemm1_amd import isa_check

MFMA = "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]"


def kernel(*lines):
    return "\n".join(["_ZN4coda1kEv:"] + list(lines) + ["\ts_endpgm", ".Lfunc_end0:"])


def nops(n):
    return [f"\ts_nop {n - 1}"] if n else []


def test_straight_line_read_too_close():
    bad = isa_check.check_asm_text(kernel(MFMA, "\tv_add_u32 v8, v9, v10",
                                          "\tv_accvgpr_read_b32 v11, a2"))
    assert len(bad) == 1 and bad[0][3] == 1


def test_straight_line_after_enough_wait_states():
    ok = isa_check.check_asm_text(kernel(MFMA, *nops(8), *nops(8), *nops(8),
                                         "\tv_accvgpr_read_b32 v11, a2"))
    assert ok == []


def test_other_registers_are_free():
    ok = isa_check.check_asm_text(kernel(MFMA, "\tv_accvgpr_write_b32 a4, v1",
                                         "\tv_accvgpr_mov_b32 a8, a5"))
    assert ok == []


def test_hazard_through_taken_branch():
    bad = isa_check.check_asm_text(kernel(
        MFMA, "\ts_cbranch_scc1 .LBB0_2",
        *nops(8), *nops(8), *nops(8), "\ts_branch .LBB0_3",
        ".LBB0_2:", "\tv_accvgpr_read_b32 v11, a1",
        ".LBB0_3:", "\ts_nop 0"))
    assert [b[2] for b in bad] == ["v_accvgpr_read_b32 v11, a1"]


def test_block_reached_only_by_distant_branch():
    ok = isa_check.check_asm_text(kernel(
        "\ts_cbranch_scc1 .LBB0_2", MFMA, *nops(8), *nops(8), *nops(8),
        "\ts_branch .LBB0_3",
        ".LBB0_2:", "\tv_accvgpr_mov_b32 a0, a252",
        ".LBB0_3:", "\ts_nop 0"))
    assert ok == []


def test_hazard_across_loop_back_edge():
    bad = isa_check.check_asm_text(kernel(
        ".LBB0_1:", "\tv_accvgpr_write_b32 a3, v1", *nops(8), *nops(8), *nops(8),
        MFMA, "\ts_cbranch_scc0 .LBB0_1"))
    assert len(bad) == 1 and bad[0][2].startswith("v_accvgpr_write_b32 a3")


def test_spill_report():
    text = "\n".join(["    .name:           _ZN4coda1aEv", "    .sgpr_spill_count: 3",
                      "    .vgpr_spill_count: 0", "    .name:           _ZN4coda1bEv",
                      "    .sgpr_spill_count: 0", "    .vgpr_spill_count: 12"])
    assert isa_check.spills(text) == [("_ZN4coda1aEv", "sgpr", 3), ("_ZN4coda1bEv", "vgpr", 12)]
