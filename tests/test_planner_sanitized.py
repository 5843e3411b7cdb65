"""The host planner (plan.cpp, partition.cpp, route.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer: a g++ build of those sources
alone is driven by the planner, partition and routing comparisons against the
oracle, on the fixed trees of those tests (zero-length nodes, a 200-node
chain, a 64-child star, the full spine tree) and on 10,000 seeded random
forests of up to 16 nodes (chains, stars, several roots, zero-length
nodes).  Runs on the CPU; skipped where g++ or its
sanitizer runtimes are absent."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_planner_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from prefix_shared_masked_amd.build import build_host_sanitized
    lib = build_host_sanitized(str(tmp_path / "libtree_plan_san.so"))
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_planner_driver.py"), lib, "10000"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=1800)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "random forests ok: 10000" in r.stdout, r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
