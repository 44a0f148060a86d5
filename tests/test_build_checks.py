"""Host-side checks of the build: the DPP wait-state scan that guards the indexer's
hand-written DPP weight broadcast, and that the indexer's generated code passes it."""
import shutil
from pathlib import Path

import pytest

from dsa_sparse_attention_indexer_amd import build

CLEAN = """
    v_max_i32_e32 v3, 0, v3
    v_mfma_f32_32x32x16_bf16 v[32:47], a[0:3], v[16:19], v[32:47]
    v_fmac_f32_dpp v5, v6, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf
"""


def test_scan_accepts_distant_writes():
    text = "    v_mov_b32_e32 v6, v7\n    s_nop 1\n" + CLEAN
    assert build.dpp_hazards(text) == []


def test_scan_flags_close_write():
    text = "    v_mov_b32_e32 v6, v7\n    v_fmac_f32_dpp v5, v6, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
    assert len(build.dpp_hazards(text)) == 1


def test_scan_flags_write_one_state_away_and_register_ranges():
    text = ("    v_add_u32_e32 v[6:7], v1, v2\n    s_nop 0\n"
            "    v_mul_f32_dpp v5, v7, v3 row_newbcast:0 row_mask:0xf bank_mask:0xf\n")
    assert len(build.dpp_hazards(text)) == 1


def test_scan_ignores_non_source_operands_and_compares():
    text = ("    v_cmp_gt_i32_e32 vcc, v6, v1\n    v_max_i32_e32 v3, 0, v3\n"
            "    v_fmac_f32_dpp v5, v6, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n")
    assert build.dpp_hazards(text) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not Path("/opt/rocm/bin/hipcc").exists(),
                    reason="needs hipcc")
def test_indexer_code_has_no_dpp_hazard():
    for src in build.DPP_SOURCES:
        build._check_dpp(src)  # raises on a hazard
