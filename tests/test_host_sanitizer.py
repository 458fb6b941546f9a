"""The planner and the C-ABI argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, no GPU): tests/host_fuzz/fuzz_capi.cpp
links plan.cpp and capi.cpp with stub launchers that check the argument blocks
they receive, and runs thousands of random problems (mostly valid, some with a
bad field) through mla_verify_plan, the run entry points and the argument
checks of the other entry points."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_absorbed_tree_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_and_argument_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "fuzz_capi")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "host_fuzz", "fuzz_capi.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "capi.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe, "4000"], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout, res.stderr[-4000:])
    assert res.returncode == 0, res.stderr[-4000:]
    assert "failures 0" in res.stdout
