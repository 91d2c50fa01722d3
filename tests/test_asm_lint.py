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


def test_spill_in_the_mfma_loop_is_flagged():
    # the tile loop (depth 2, holds the MFMAs) with a zeroing loop nested in it (depth 3) inside the
    # segment loop (depth 1): spills in the tile loop or the loop nested in it are flagged, spills in
    # the segment loop or outside every loop are not
    body = (".LBB2_1:  ; =>This Loop Header: Depth=1\n"
            "\tscratch_load_dword v3, off, off offset:4\n"
            ".LBB2_2:  ;   Parent Loop BB2_1 Depth=1\n"
            "           ; =>  This Loop Header: Depth=2\n"
            "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n"
            "\tscratch_load_dwordx4 v[18:21], off, off\n"
            ".LBB2_3:  ;   Parent Loop BB2_2 Depth=2\n"
            "           ; =>    This Inner Loop Header: Depth=3\n"
            "\tscratch_load_dword v9, off, off offset:8\n"
            "; %bb.4:  ;   in Loop: Header=BB2_2 Depth=2\n"
            "\tscratch_load_dword v10, off, off offset:12\n"
            ".LBB2_5:\n"
            "\tscratch_store_dword off, v3, off\n")
    problems = _lint(body)
    assert len(problems) == 3
    assert "scratch_load_dwordx4" in problems[0] and "v9" in problems[1] and "v10" in problems[2]


def test_spill_in_a_loop_without_mfmas_is_allowed():
    body = (".LBB2_1:  ; =>This Loop Header: Depth=1\n"
            "\tscratch_load_dword v3, off, off offset:4\n"
            "\tv_add_u32_e32 v1, v2, v3\n")
    assert _lint(body) == []


def test_spill_outside_loops_is_allowed():
    body = "\tscratch_store_dword off, v3, off\n.LBB2_1:  ; =>This Loop Header: Depth=1\n\tv_add_u32_e32 v1, v2, v3\n"
    assert _lint(body) == []


def _build_module():
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from mla_paged_kv_decode_amd import build
    return build


def test_spill_gate_covers_the_default_instantiations():
    b = _build_module()
    pre = "_ZN3mla12_GLOBAL__N_120mla_split_kv_partialI"
    gated = [pre + "Li2ELb1ELb0ELb1EEEvNS_13PartialParamsE",   # E4M3, pages >= a tile, no window
             pre + "Li1ELb1ELb0ELb0EEEvNS_13PartialParamsE",   # bf16, own rows
             pre + "Li1ELb1ELb1ELb1EEEvNS_13PartialParamsE",   # bf16, cross-wave, window
             pre + "Li3ELb1ELb0ELb1EEEvNS_13PartialParamsE",   # fp16
             pre + "Li4ELb1ELb0ELb0EEEvNS_13PartialParamsE",   # bf16 q over E4M3
             "_ZN3mla12_GLOBAL__N_116mla_combine_wideILb1EEEvNS_13CombineParamsE",
             "_ZN3mla12_GLOBAL__N_115mla_kv_pack_fp8ENS_10PackParamsE"]
    free = [pre + "Li2ELb1ELb1ELb1EEEvNS_13PartialParamsE",     # E4M3 four-wave kernel with a window
            pre + "Li2ELb0ELb0ELb1EEEvNS_13PartialParamsE",     # E4M3 over short pages
            pre + "Li1ELb0ELb0ELb0EEEvNS_13PartialParamsE",     # bf16 over short pages
            "_ZN3mla12_GLOBAL__N_122mla_split_kv_fp8_rolesILb1ELb0EEEvNS_13PartialParamsE"]
    assert all(b.must_not_spill(k) for k in gated)
    assert not any(b.must_not_spill(k) for k in free)
    res = {k: {"VGPRs Spill": 0} for k in gated + free}
    assert b.spill_gate(res) == []
    res[gated[0]]["VGPRs Spill"] = 3
    res[free[0]]["VGPRs Spill"] = 15
    bad = b.spill_gate(res)
    assert len(bad) == 1 and gated[0] in bad[0]


def test_built_library_has_no_spills_in_the_gated_kernels():
    b = _build_module()
    path = os.path.join(os.path.dirname(b.LIB), "kernel_resources.txt")
    if not os.path.exists(path):
        import pytest
        pytest.skip("library not built here (kernel_resources.txt is written by the build)")
    rows = {}
    for line in open(path):
        name, _, rest = line.partition(": ")
        fields = dict(kv.split("=") for kv in rest.split())
        rows[name] = {"VGPRs Spill": int(fields["vgpr_spill"])}
    assert any(b.must_not_spill(k) for k in rows)
    assert b.spill_gate(rows) == []
