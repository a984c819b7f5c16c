"""The encoder's inline-assembly stores against the gfx950 rule that a
vector-memory instruction reading a VALU-written SGPR needs five wait
states, checked in the assembly of the current sources (hipcc
cross-compiles; no GPU needed)."""
import os
import shutil

import pytest

from tests import asm_hazards as H
from tests import asm_prefetch as A


@pytest.mark.slow
def test_encoder_stores_clear_of_valu_sgpr_writes(tmp_path):
    if not os.path.exists(shutil.which("hipcc") or "/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    asm = str(tmp_path / "cg_kernels.s")
    A.compile_asm(asm)
    lines = open(asm).read().split("\n")
    for sym in H.ENCODERS:
        n, problems = H.check_kernel(lines, sym)
        assert n >= 96, (sym, n)  # three batches of 16 tokens, two stores each, at least
        assert not problems, (sym, problems[:4])


STORE = "buffer_store_short v4, v7, s[4:7], s85 idxen"


def test_checker_flags_readfirstlane_into_offset():
    lines = ["v_readfirstlane_b32 s85, v3", "s_and_saveexec_b64 s[2:3], s[4:5]", STORE]
    n, p = H.check_lines(lines)
    assert n == 1 and len(p) == 1 and "[85]" in p[0][1]


def test_checker_flags_compare_into_descriptor():
    lines = ["v_cmp_gt_u32_e64 s[6:7], v1, v2", "s_mov_b32 s9, 0", STORE]
    n, p = H.check_lines(lines)
    assert len(p) == 1


def test_checker_flags_label_in_window():
    lines = ["s_lshl_b32 s85, s49, 1", ".LBB0_3:", "s_and_saveexec_b64 s[2:3], s[8:9]", STORE]
    n, p = H.check_lines(lines)
    assert len(p) == 1 and "label" in p[0][1]


def test_checker_accepts_scalar_offset_and_distant_valu():
    lines = ["v_readfirstlane_b32 s85, v3", "s_nop 4", "s_lshl_b32 s85, s49, 1",
             "s_and_saveexec_b64 s[2:3], s[10:11]", STORE]
    n, p = H.check_lines(lines)
    assert n == 1 and not p
    lines = ["v_cmp_gt_u32_e64 s[54:55], v74, v7", "s_bcnt1_i32_b64 s56, s[54:55]",
             "s_sub_i32 s49, s49, s56", "s_lshl_b32 s85, s49, 1", "s_and_saveexec_b64 s[56:57], s[54:55]", STORE]
    n, p = H.check_lines(lines)
    assert not p
