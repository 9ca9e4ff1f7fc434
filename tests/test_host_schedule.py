"""Host logic of the C library, built with g++ (no HIP): the GDN tree stash
schedule and the conv window-source table (tests/host/schedule_check.cpp)."""
import os
import shutil
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "hybrid_recurrent_state_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tree_schedule_and_window_sources():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "schedule_check")
        cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=address,undefined", "-I", CSRC,
               os.path.join(ROOT, "tests", "host", "schedule_check.cpp"), os.path.join(CSRC, "validate.cpp"),
               "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True)
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert res.returncode == 0, res.stdout + res.stderr
        assert res.stdout.startswith("OK")
