"""bench.py's command line without a GPU: more than one GPU is refused with a
message and exit status 2 before anything touches a device."""
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")
