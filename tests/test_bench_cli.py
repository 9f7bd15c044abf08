"""bench.py's command line on the host (CPU only): the path is single-GPU, so a
multi-GPU request exits with status 2 and says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr + r.stdout
    assert r.stdout.strip() == ""   # no JSON line for a refused run
