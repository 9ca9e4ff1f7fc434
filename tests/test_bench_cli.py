"""bench.py's command-line contract on the host: more than one GPU is refused
with a message before anything touches a device."""
import os
import subprocess
import sys

from tests.conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""
