"""bench.py's command line on a machine without a GPU: a request for more
than one GPU ends with a message and exit status 2 before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stdout[-500:], r.stderr[-500:])
    assert "one GPU only" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")
