"""The build-time assembly checks (mla_paged_kv_decode_amd/asm_lint.py) on small hand-written listings:
each rule must flag its hazard and stay quiet on the safe form."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "mla_paged_kv_decode_amd"))
import asm_lint  # noqa: E402

NAME = "_ZN3mla12_GLOBAL__N_120mla_split_kv_partialILi2ELb1EEEvNS_13PartialParamsE"


def _lint(body: str) -> list:
    report = asm_lint.lint(f"{NAME}:\n{body}\n")
    assert list(report) == [NAME]
    return report[NAME]


def test_mfma_result_read_too_early_is_flagged():
    bad = "\tv_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[32:39], v[56:63], 0, v252, v252\n\tv_max_f32_e32 v0, v16, v17"
    assert any("after the MFMA" in p for p in _lint(bad))
    good = bad.replace("\tv_max_f32", "\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_max_f32")
    assert _lint(good) == []


def test_mfma_reading_fresh_valu_result_is_flagged():
    bad = "\tv_and_b32_e32 v56, -1, v56\n\tv_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[32:39], v[56:63], 0, v252, v252"
    assert any("written by VALU" in p for p in _lint(bad))
    good = bad.replace("\tv_mfma", "\ts_nop 2\n\tv_mfma")
    assert _lint(good) == []


def test_mfma_accumulator_chain_is_not_a_hazard():
    chain = ("\tv_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[32:39], v[56:63], 0, v252, v252\n"
             "\tv_mfma_scale_f32_32x32x64_f8f6f4 v[16:31], v[40:47], v[64:71], v[16:31], v252, v252")
    assert _lint(chain) == []


def test_spill_in_innermost_loop_is_flagged():
    body = (".LBB2_1:  ; =>This Loop Header: Depth=1\n"
            "\tscratch_load_dword v3, off, off offset:4\n"
            ".LBB2_2:  ;   Parent Loop BB2_1 Depth=2\n"
            "\tscratch_load_dwordx4 v[18:21], off, off\n"
            ".LBB2_3:\n"
            "\tscratch_store_dword off, v3, off\n")
    problems = _lint(body)
    assert len(problems) == 1 and "scratch_load_dwordx4" in problems[0]


def test_spill_outside_loops_is_allowed():
    body = "\tscratch_store_dword off, v3, off\n.LBB2_1:  ; =>This Loop Header: Depth=1\n\tv_add_u32_e32 v1, v2, v3\n"
    assert _lint(body) == []
