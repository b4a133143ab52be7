"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "gpus" in r.stderr.lower() or "gpu" in r.stderr.lower()
    assert r.stdout.strip() == ""
