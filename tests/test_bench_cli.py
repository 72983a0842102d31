"""bench.py's command line on the CPU: it measures one GPU only and refuses a
request for more before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
