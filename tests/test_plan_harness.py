"""The library's launch planning (csrc/fa2_plan.h: the key split of small
prefill grids, the split-KV chunking, workspace sizes and strided-tensor
checks) built on the CPU with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and run over a grid of shapes and device sizes
(tests/host/plan_harness.cpp says what it checks). No GPU involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_tiled_amd", "csrc")
HARNESS = os.path.join(ROOT, "tests", "host", "plan_harness.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_harness_sanitized(tmp_path):
    exe = str(tmp_path / "plan_harness")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
         "-Wno-unused-function", "-Werror", "-I", CSRC, "-o", exe, HARNESS],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert run.stdout.startswith("plan harness OK"), run.stdout
