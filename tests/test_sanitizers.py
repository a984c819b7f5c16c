"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (no GPU work): tests/sanitize/
oracle_harness.c drives every oracle entry point on small seeded inputs and
damaged records; tests/sanitize/host_harness.cpp drives the library's
argument checks, size queries, dispatch planner and launch setup with the
kernel launchers stubbed out. Both must finish clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, env=None, timeout=300):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return p.returncode, p.stdout + p.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    rc, out = run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                   os.path.join(ROOT, "oracle", "cg_oracle.c"), os.path.join(HERE, "oracle_harness.c"),
                   "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = run([exe], env=ENV)
    assert rc == 0 and "all checks passed" in out, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_host_code_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_harness")
    # sanitizers on the host half of the build only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    rc, out = run([HIPCC, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "--offload-arch=gfx950", *san,
                   "-x", "hip", os.path.join(ROOT, "kv_cache_compression_encode_amd", "csrc", "cg_api.cpp"),
                   os.path.join(HERE, "host_harness.cpp"), "-o", exe])
    assert rc == 0, out
    # the HIP runtime's own allocations are not this code's: leak checks off
    rc, out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert rc == 0 and "all checks passed" in out, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
