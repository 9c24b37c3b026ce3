"""The host partitioner under address and undefined-behaviour sanitizers: random batches,
valid and with planted defects, through build_schedule (tests/host_fuzz/fuzz_schedule.cpp).
Accepted schedules must keep every unit, workspace row and merge inside its bounds;
planted defects must be rejected with a message."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_attention_serving_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host_fuzz", "fuzz_schedule.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_partitioner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "fuzz_schedule")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror", "-I", CSRC, SRC,
           os.path.join(CSRC, "partition.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "1500"], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="abort_on_error=0"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok 1500 ")
