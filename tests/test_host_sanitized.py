"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/native/planner_check.cpp links the library's pure-C++ planner (validation, page
layouts of one, several and growable layers, the attention work list, the plan serialiser)
and checks its invariants on random shapes; here it is compiled with g++ and both sanitizers
(no GPU code in the build) and must finish clean."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_aware_paged_segpaged_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "planner_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "planner_check.cpp"),
           os.path.join(CSRC, "planner.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for seed in (1, 2):
        res = subprocess.run([exe, "150", str(seed)], capture_output=True, text=True, env=env,
                             timeout=600)
        out = res.stdout + res.stderr
        assert res.returncode == 0, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
        assert "0 failures" in res.stdout
