"""Host-side check of the device-assembly scan the build runs over sources
with inline asm (a transcendental VALU op followed directly by inline asm
that touches its registers)."""
from evicted_kv_cache_amd.asm_check import scan

HEAD = "_Zkernel:\n"


def _asm(*body):
    return HEAD + "\n".join(body) + "\n"


def test_flags_read_of_fresh_result():
    text = _asm("\tv_exp_f32_e32 v18, v18", "\t;;#ASMSTART", "\tv_fma_mix_f32 v21, v26, v18, 0 op_sel_hi:[1,0,0]",
                "\t;;#ASMEND")
    hits = scan(text)
    assert len(hits) == 1 and "v_exp_f32_e32 v18, v18" in hits[0]


def test_flags_overwrite_of_source():
    # the asm overwrites v2 while v_exp_f32 still reads it
    text = _asm("\tv_exp_f32_e32 v77, v2", "\t;;#ASMSTART", "\tv_fma_mix_f32 v2, v22, v79, 0 op_sel_hi:[1,0,0]",
                "\t;;#ASMEND")
    assert len(scan(text)) == 1


def test_flags_overwrite_of_result_and_register_ranges():
    text = _asm("\tv_rcp_f32_e32 v5, v9", "\t;;#ASMSTART", "\tv_dot2_f32_f16 v5, v[0:1], v3, 0", "\t;;#ASMEND",
                "\tv_sqrt_f32_e32 v1, v4", "\t;;#ASMSTART", "\tv_dot2_f32_f16 v8, v[0:1], v3, 0", "\t;;#ASMEND")
    hits = scan(text)
    assert len(hits) == 2


def test_wait_state_or_unrelated_registers_pass():
    text = _asm(
        # an s_nop between: one wait state
        "\tv_exp_f32_e32 v18, v18", "\ts_nop 0", "\t;;#ASMSTART", "\tv_fma_mix_f32 v21, v26, v18, 0", "\t;;#ASMEND",
        # a compiler-emitted instruction between
        "\tv_exp_f32_e32 v30, v31", "\tv_mov_b32_e32 v40, v41", "\t;;#ASMSTART", "\tv_fma_mix_f32 v31, v30, v1, 0",
        "\t;;#ASMEND",
        # asm right after, but on other registers
        "\tv_log_f32_e32 v50, v51", "\t;;#ASMSTART", "\tv_fma_mix_f32 v52, v53, v54, v55", "\t;;#ASMEND",
        # compiler code right after (the compiler handles its own hazards)
        "\tv_exp_f32_e32 v60, v61", "\tv_mul_f32_e32 v61, v60, v60")
    assert scan(text) == []


def test_comments_and_labels_are_skipped():
    text = _asm("\tv_exp_f32_e32 v7, v8", "; %bb.3:", ".LBB0_4:", "\t;;#ASMSTART", "\tv_fma_mix_f32 v9, v7, v1, 0",
                "\t;;#ASMEND")
    assert len(scan(text)) == 1
