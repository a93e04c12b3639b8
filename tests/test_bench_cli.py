"""bench.py's command line without a GPU: a request for more than one GPU is
refused with a message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2 and "one GPU" in res.stderr
