"""bench.py's command line on the CPU: more than one GPU is refused with a message, before anything touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n), "--steps", "1"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""  # no JSON line
