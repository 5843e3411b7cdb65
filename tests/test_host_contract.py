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


def test_binding_checks_buffers_on_the_host():
    """The binding rejects, before any launch, tensors whose shape, dtype,
    layout or device differ from what the kernels assume (they take raw
    pointers), malformed workspaces, and decode span tables that leave the
    K/V rows or exceed max_len."""
    import numpy as np
    import pytest
    import torch
    import prefix_shared_masked_amd as pkg
    cpu = torch.device("cpu")
    x = torch.zeros(4, 2, 8)
    with pytest.raises(ValueError, match="shape"):
        pkg._need(x, "dq", (4, 2, 16), torch.float32, cpu)
    with pytest.raises(ValueError, match="dtype"):
        pkg._need(x, "dq", (4, 2, 8), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        pkg._need(x.transpose(0, 1), "dq", (2, 4, 8), torch.float32, cpu)
    with pytest.raises(ValueError, match="live on"):
        pkg._need(x, "dq", (4, 2, 8), torch.float32, cpu)  # a CPU tensor is never accepted
    with pytest.raises(ValueError, match="uint8"):
        pkg._workspace(64, cpu, torch.zeros(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous uint8"):
        pkg._workspace(64, cpu, torch.zeros(128, dtype=torch.uint8)[::2])
    with pytest.raises(ValueError, match="live on"):
        pkg._workspace(64, cpu, torch.zeros(64, dtype=torch.uint8))
    i32 = lambda a: torch.tensor(np.asarray(a, np.int32))
    pkg._check_spans(i32([0, 1, 3]), i32([[0, 10], [10, 5], [20, 4]]), 24, 10)
    with pytest.raises(ValueError, match="outside"):
        pkg._check_spans(i32([0, 1, 3]), i32([[0, 10], [10, 5], [20, 5]]), 24, 10)
    with pytest.raises(ValueError, match="outside"):
        pkg._check_spans(i32([0, 1]), i32([[-1, 3]]), 24, 10)
    with pytest.raises(ValueError, match="max_len"):
        pkg._check_spans(i32([0, 1, 3]), i32([[0, 10], [10, 5], [20, 4]]), 24, 8)
    with pytest.raises(ValueError, match="span_ptr"):
        pkg._check_spans(i32([0, 2, 1]), i32([[0, 1], [1, 1]]), 24, 10)
    pkg._check_spans(i32([0, 0, 1]), i32([[3, 2]]), 24, 10)  # an empty item is fine


def test_library_global_state_is_the_documented_state():
    """The header lists the library's only global mutable state: the scratch
    array of the allocation-free decode call with its per-device address
    table and mutex.  List the writable data objects the built library defines itself
    (kernel launch stubs, which are functions, and the compiler's and HIP
    runtime's own registration objects excluded)."""
    lib = os.path.join(ROOT, "prefix_shared_masked_amd", "libtree_attn.so")
    out = subprocess.run(["nm", "-C", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    objs = set()
    for line in out.splitlines():
        parts = line.split(maxsplit=2)
        if len(parts) < 3 or parts[1] not in "bBdD":
            continue
        name = parts[2]
        # (a kernel stub whose argument types the demangler does not know stays mangled: "_Z...")
        if name.endswith(")") or name.startswith(("__", "_Z", "_DYNAMIC", "_GLOBAL_OFFSET_TABLE_", "DW.ref.")):
            continue
        objs.add(name)
    assert objs == {"scratch", "(anonymous namespace)::g_scratch_mu", "(anonymous namespace)::g_scratch_ptr"}, objs


def test_library_links_no_vendor_math_library():
    """Every kernel is the library's own: the built library links no BLAS
    (hipBLASLt, rocBLAS) or other vendor math library."""
    lib = os.path.join(ROOT, "prefix_shared_masked_amd", "libtree_attn.so")
    out = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    needed = [l for l in out.splitlines() if "(NEEDED)" in l]
    assert needed and not any(x in l.lower() for l in needed for x in ("blas", "miopen", "rocsolver", "hipfft")), needed
