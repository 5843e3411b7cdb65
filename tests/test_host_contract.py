"""Host-side contracts: bench.py refuses more than one GPU with a message
before any device work (this library runs on one GPU and has no collectives
between GPUs), and the Python binding has no CPU fallback when the HIP
library is absent."""
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


def test_missing_library_fails_loudly():
    """No CPU fallback: with the HIP library absent, the first call raises."""
    code = (
        "import numpy as np, prefix_shared_masked_amd as pkg\n"
        "pkg._LIB_PATH = '/nonexistent/libtree_attn.so'\n"
        "try:\n"
        "    pkg.tree_plan(np.array([-1, 0], np.int32), np.array([4, 3], np.int32))\n"
        "except pkg.TreeAttnError as e:\n"
        "    print('raised', e)\n"
        "else:\n"
        "    print('returned')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised"), r.stdout
