"""The decoder's inline-assembly stream prefetches, checked in the gfx950
assembly of the current sources (no GPU needed; hipcc cross-compiles)."""
import os
import shutil

import pytest

from tests import asm_prefetch as A


@pytest.mark.slow
def test_no_prefetch_register_used_in_flight(tmp_path):
    if not os.path.exists(shutil.which("hipcc") or "/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    asm = str(tmp_path / "cg_kernels.s")
    A.compile_asm(asm)
    res = A.check_all(asm)
    assert set(res) == set(A.DECODERS)
    for kernel, (hazards, refills) in res.items():
        # the prefetches were found: every decoder refills its rings from them
        assert refills, kernel
        assert not hazards, (kernel, hazards[:4])


def _fake(body):
    head = ["_Zfake:", "\ts_mov_b32 s0, 0"]
    return head + ["\t" + l if not l.startswith(".LBB") else l for l in body] + ["\ts_endpgm", ".Lfunc_end0:"]


LOAD = ["s_nop 4", "buffer_load_dword v6, v10, s[8:11], 0 offen"]


def test_checker_flags_copy_before_wait():
    lines = _fake(LOAD + ["v_mov_b32_e32 v7, v6", "s_waitcnt vmcnt(0)"])
    hz, _ = A.check_kernel(lines, "_Zfake")
    assert len(hz) == 1 and "v_mov_b32_e32 v7, v6" in hz[0][2]


def test_checker_flags_reuse_before_wait():
    lines = _fake(LOAD + ["v_add_u32_e32 v6, v1, v2", "s_waitcnt vmcnt(0)"])
    hz, _ = A.check_kernel(lines, "_Zfake")
    assert len(hz) == 1 and hz[0][2].startswith("overwritten")


def test_checker_accepts_copy_after_covering_wait():
    # vmcnt(1) with one store issued after the load: the load is complete
    lines = _fake(LOAD + ["buffer_store_short v1, v3, s[12:15], s4 offen", "s_waitcnt vmcnt(1)",
                          "v_mov_b32_e32 v7, v6"])
    hz, _ = A.check_kernel(lines, "_Zfake")
    assert hz == []
    # vmcnt(1) with nothing issued after it: still in flight
    lines = _fake(LOAD + ["s_waitcnt vmcnt(1)", "v_mov_b32_e32 v7, v6", "s_waitcnt vmcnt(0)"])
    hz, _ = A.check_kernel(lines, "_Zfake")
    assert len(hz) == 1


def test_checker_follows_constant_flags():
    # the copy sits on a path the flag s[4:5] = 0 rules out
    body = LOAD + ["s_mov_b64 s[4:5], 0", "s_and_b64 vcc, exec, s[4:5]", "s_cbranch_vccz .LBB0_2",
                   "v_mov_b32_e32 v7, v6", ".LBB0_2:", "s_waitcnt vmcnt(0)"]
    hz, _ = A.check_kernel(_fake(body), "_Zfake")
    assert hz == []
    body[2] = "s_mov_b64 s[4:5], -1"
    hz, _ = A.check_kernel(_fake(body), "_Zfake")
    assert len(hz) == 1
