"""The step planner (csrc/plan.cpp: validation, size classes, descriptor
order, tile prefixes, per-XCD tile ranges, workspace layout) built on its own
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, with its
internal bounds checks on, and run over thousands of random batches by
tests/native/plan_check.cpp.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_step_02_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-DMUON_PLAN_CHECKS",
           "-D_GLIBCXX_ASSERTIONS", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "native", "plan_check.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), "3000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
