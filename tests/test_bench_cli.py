"""bench.py's command line on the host: it measures one GPU only, so any
--gpus above 1 exits with status 2 and says so, before touching a GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mode", ["step", "ingest", "sweep", "gemv"])
def test_more_than_one_gpu_is_refused(mode):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                          "--mode", mode], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_help_lists_the_contract_flags():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--mode"):
        assert flag in res.stdout
