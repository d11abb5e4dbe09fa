"""The build's scan for DPP read-after-write hazards (our own generated code)."""
from bayesian_memory_scan_amd import _build


def test_hazard_found_without_wait_states():
    asm = ("_Zk:\n"
           "\tv_mul_f32_e32 v5, v1, v2\n"
           "\tv_fmac_f32_dpp v6, v5, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf\n")
    assert len(_build.dpp_hazards(asm)) == 1


def test_hazard_one_instruction_apart():
    asm = ("_Zk:\n"
           "\tv_mul_f32_e32 v5, v1, v2\n"
           "\tv_add_f32_e32 v9, v1, v2\n"
           "\tv_fmac_f32_dpp v6, v5, v7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n")
    assert len(_build.dpp_hazards(asm)) == 1


def test_padded_or_unrelated_code_passes():
    asm = ("_Zk:\n"
           "\tv_mul_f32_e32 v5, v1, v2\n"
           "\ts_nop 1\n"
           "\tv_fmac_f32_dpp v6, v5, v7 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
           "\tv_mul_f32_e32 v8, v1, v2\n"
           "\tv_fmac_f32_dpp v6, v5, v8 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
           "\tds_read_b32 v11, v3\n"
           "\ts_waitcnt lgkmcnt(0)\n"
           "\tv_fmac_f32_dpp v6, v11, v8 row_newbcast:2 row_mask:0xf bank_mask:0xf\n")
    assert _build.dpp_hazards(asm) == []


def test_built_library_is_clean():
    """Every source of the library, as last built, passed the scan."""
    import os
    for src in _build.SOURCES:
        asm = os.path.join(_build.BUILD, src.replace(".hip", "-hip-amdgcn-amd-amdhsa-gfx950.s"))
        if os.path.exists(asm):
            assert _build.dpp_hazards(open(asm).read()) == [], src
