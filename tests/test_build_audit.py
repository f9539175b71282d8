"""The build refuses gfx950 code in which the compiler touched the AGPRs that hold the output
accumulator on the waves that hold it, placed a VALU write of an inline-asm MFMA operand inside
the hazard window, used m0 (which the LDS-DMA gathers set) or gave a kernel private scratch
memory.  These tests feed the checks small hand-written assembly listings."""

from mla_tree_verify_mlaverify_amd import build

HEAD = "k:\n"


def asm(*lines):
    return HEAD + "".join("\t" + l + "\n" if not l.startswith(";;") and not l.endswith(":") else l + "\n" for l in lines)


def test_agpr_audit_accepts_asm_only_use():
    text = asm(";;#ASMSTART", "v_accvgpr_write_b32 a0, 0", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
               ";;#ASMEND", "v_add_f32_e32 v1, v2, v3")
    assert build.audit_agprs(text) == []


def test_agpr_audit_flags_compiler_agpr_use():
    text = asm("v_accvgpr_write_b32 a3, v7", ";;#ASMSTART", "v_accvgpr_read_b32 v1, a0", ";;#ASMEND")
    bad = build.audit_agprs(text)
    assert len(bad) == 1 and "a3, v7" in bad[0]


MARK = [";;#ASMSTART", "; " + build.HELPER_MARK, ";;#ASMEND"]


def test_agpr_audit_allows_the_helper_region_only():
    # the helper waves hold no accumulator: AGPR uses past the marker pass, the same use on
    # the path of the compute waves does not
    helper = asm("s_cmp_lt_u32 s0, 2", "s_cbranch_scc1 .LBB0_2", "; %bb.1:", *MARK,
                 "global_load_dwordx4 a[0:3], v[20:21], off", "v_accvgpr_read_b32 v1, a5", "s_endpgm",
                 ".LBB0_2:", "v_add_f32_e32 v1, v2, v3", "s_endpgm")
    assert build.audit_agprs(helper) == []
    compute = helper.replace("v_add_f32_e32 v1, v2, v3", "v_accvgpr_write_b32 a7, v2")
    bad = build.audit_agprs(compute)
    assert len(bad) == 1 and "a7, v2" in bad[0]


def test_agpr_audit_checks_code_before_the_marker_and_shared_blocks():
    # in the marker's block, the code above the marker is audited; so is a block that the
    # helper region branches back into when the compute path reaches it too
    before = asm("s_cbranch_scc1 .LBB0_2", "; %bb.1:", "v_accvgpr_write_b32 a0, v2", *MARK, "s_endpgm",
                 ".LBB0_2:", "s_endpgm")
    assert len(build.audit_agprs(before)) == 1
    shared = asm("s_cbranch_scc1 .LBB0_2", "; %bb.1:", *MARK, "v_accvgpr_write_b32 a1, v2", "s_branch .LBB0_3",
                 ".LBB0_2:", "v_add_f32_e32 v1, v2, v3", ".LBB0_3:", "v_accvgpr_read_b32 v4, a1", "s_endpgm")
    bad = build.audit_agprs(shared)
    assert len(bad) == 1 and "v4, a1" in bad[0]


def test_agpr_audit_scopes_by_symbol():
    # each function is walked from its own entry; block comments do not start a function
    text = ("_ZN3mlv4foo:\n; %bb.0:\n\tv_add_f32_e32 v1, v2, v3\n\ts_endpgm\n"
            "_ZN3mlv9k_partialILb0ELb0ELb1EEEvNS_11PartialArgsE:\n; %bb.0:\n\tv_accvgpr_write_b32 a7, v2\n")
    bad = build.audit_agprs(text)
    assert len(bad) == 1 and bad[0].startswith("_ZN3mlv9k_partial") and "a7, v2" in bad[0]


def test_m0_audit():
    ok = asm(";;#ASMSTART", "s_add_u32 m0, s4, 0x1000", "s_nop 0", "global_load_lds_dwordx4 v[2:3], off", ";;#ASMEND",
             "v_add_f32_e32 v1, v2, v3")
    assert build.audit_m0(ok) == []
    bad = asm("s_mov_b32 m0, s5", "v_readlane_b32 s6, v1, m0")
    assert len(build.audit_m0(bad)) == 2


def test_kernel_resources_reads_scratch_and_registers():
    meta = ("  - .name: k_a\n    .private_segment_fixed_size: 0\n    .vgpr_count: 476\n"
            "  - .name: k_b\n    .private_segment_fixed_size: 56\n    .vgpr_count: 504\n")
    assert build.kernel_resources(meta) == [("k_a", 0, 476), ("k_b", 56, 504)]


def test_mfma_audit_flags_valu_write_of_operand():
    text = asm("v_mov_b32_e32 v4, v10", ";;#ASMSTART",
               "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    assert len(build.audit_mfma_operands(text)) == 1


def test_mfma_audit_accepts_distant_or_unrelated_writes():
    far = asm("v_mov_b32_e32 v4, v10", "v_add_u32_e32 v20, v21, v22", "v_add_u32_e32 v23, v21, v22", ";;#ASMSTART",
              "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    nop = asm("v_mov_b32_e32 v4, v10", "s_nop 1", ";;#ASMSTART",
              "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    other = asm("v_mov_b32_e32 v40, v10", ";;#ASMSTART",
                "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    lds = asm("ds_read_b128 v[2:5], v1", "s_waitcnt lgkmcnt(0)", ";;#ASMSTART",
              "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    for text in (far, nop, other, lds):
        assert build.audit_mfma_operands(text) == [], text


def test_mfma_audit_flags_label_in_window():
    text = asm(".LBB0_3:", ";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND")
    assert len(build.audit_mfma_operands(text)) == 1
