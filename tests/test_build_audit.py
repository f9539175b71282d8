"""The build refuses gfx950 code in which the compiler touched the AGPRs that hold the output
accumulator, or placed a VALU write of an inline-asm MFMA operand inside the hazard window.
These tests feed the two checks small hand-written assembly listings."""

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


def test_agpr_audit_scopes_by_symbol_not_block_comment():
    # the waves that run the gather helper hold no accumulator, so its AGPR uses pass; a block
    # comment inside it ("; %bb.N:") does not end it, and the next symbol is audited again
    text = ("_ZN3mlv13gather_helperILb0EEEvPKc:\n; %bb.46:\n\tglobal_load_dwordx4 a[0:3], v[20:21], off\n"
            ".LBB3_2:\n\tv_accvgpr_read_b32 v1, a5\n"
            "_ZN3mlv9k_partialILb0ELb0ELb1EEEvNS_11PartialArgsE:\n; %bb.0:\n\tv_accvgpr_write_b32 a7, v2\n")
    bad = build.audit_agprs(text)
    assert len(bad) == 1 and bad[0].startswith("_ZN3mlv9k_partial") and "a7, v2" in bad[0]


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
