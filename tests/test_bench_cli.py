"""bench.py's command-line contract on the host: more than one GPU is refused
with a message before any device work (this library runs on one GPU and has
no collectives between GPUs)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""
