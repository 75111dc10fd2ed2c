"""The host planners under AddressSanitizer and UBSan: tests/host_fuzz/
planner_fuzz.cpp drives the decode, static, worker-count and prefill planners
over random batches, each plan written into a buffer of exactly the size its
size query returned; the planner sources are compiled with g++ for the host
alone (kernel launches stubbed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "load_balanced_paged_step_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_planners_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "planner_fuzz"
    srcs = [os.path.join(ROOT, "tests", "host_fuzz", "planner_fuzz.cpp"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(CSRC, "prefill_api.cpp"), os.path.join(CSRC, "prologue_api.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), *srcs, "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    # the environment is passed on as it is; ASan is told not to insist on
    # coming first among the loaded libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "fuzzed" in run.stdout
