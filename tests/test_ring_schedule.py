"""The attention kernel's LDS ring schedule (tree_masked_verification_amd/csrc/
ring_schedule.hpp) replayed on the host: the header's own compile-time replay must hold
and a multi-wave timing model (tests/ring_schedule_model.cpp) with random copy latencies
must never read a ring group before its copies landed nor refill a group still being read."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "tree_masked_verification_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_ring_schedule_model(tmp_path):
    exe = str(tmp_path / "ring_model")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "ring_schedule_model.cpp"), "-o", exe],
                   check=True)
    out = subprocess.run([exe], check=False, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
