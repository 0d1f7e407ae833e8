"""The host-side round planner under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

round.cpp is compiled with g++ (host code only, no GPU code involved) together
with tests/native/round_plan_sanitize.cpp, which plans seeded random rounds,
checks every plan's invariants and drives the error paths; any invalid memory
access, leak or undefined operation makes the run fail.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "collective_kv_cache_amd", "csrc", "round.cpp")
DRIVER = os.path.join(ROOT, "tests", "native", "round_plan_sanitize.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_round_planner_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "round_plan_sanitize")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include")]
    build = subprocess.run(["g++", *flags, SRC, DRIVER, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "400"], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok 400 rounds" in run.stdout
