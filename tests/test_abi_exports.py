"""The built library loads without a GPU and exports every call that
include/tree_attn.h declares; argument validation that happens before any
launch is checked without touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

import prefix_shared_masked_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ta_status|void|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("tree_plan", "tree_plan_view", "tree_plan_device_bytes", "tree_plan_upload", "tree_plan_free",
              "tree_attn_ws_bytes", "tree_attn_fwd", "tree_attn_bwd", "tree_nll_ws_bytes", "tree_weighted_nll",
              "tree_decode_ws_bytes", "tree_decode_splitkv", "ta_status_string", "tree_plan_ex",
              "tree_partition", "tree_partition_view", "tree_partition_plan", "tree_partition_device_bytes",
              "tree_partition_upload", "tree_partition_free", "tree_partition_ws_bytes", "tree_partition_fwd",
              "tree_partition_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = pkg.load_library()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pkg.library_path()], capture_output=True, text=True)
    if out.returncode == 0:
        exported = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
        for n in declared_functions():
            assert n in exported, n


def test_status_strings():
    L = pkg.load_library()
    for code in range(7):
        assert L.ta_status_string(code)
    assert L.ta_status_string(99) == b"unknown status"


def test_validation_before_launch():
    """Calls that are invalid on their face return before touching a device."""
    L = pkg.load_library()
    plan = pkg.tree_plan([-1], [8])
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    # null dplan
    assert L.tree_attn_fwd(plan.handle, None, 1, fake, fake, fake, 4, 2, 128, 0.0, 0.0, fake, fake, None, 0,
                           None) == 1
    # Hq not a multiple of Hkv
    assert L.tree_attn_fwd(plan.handle, fake, 1, fake, fake, fake, 3, 2, 128, 0.0, 0.0, fake, fake, None, 0,
                           None) == 1
    # bf16 needs d = 128; fp32 takes 64 or 128
    assert L.tree_attn_fwd(plan.handle, fake, 1, fake, fake, fake, 4, 2, 64, 0.0, 0.0, fake, fake, None, 0,
                           None) == 5
    assert L.tree_attn_fwd(plan.handle, fake, 0, fake, fake, fake, 4, 2, 96, 0.0, 0.0, fake, fake, None, 0,
                           None) == 5
    # RoPE needs a workspace
    assert L.tree_attn_fwd(plan.handle, fake, 1, fake, fake, fake, 4, 2, 128, 0.0, 10000.0, fake, fake, None, 0,
                           None) == 4
    assert L.tree_attn_bwd(plan.handle, fake, 1, fake, fake, fake, fake, fake, fake, 4, 2, 128, 0.0, 0.0, fake,
                           fake, fake, None, 0, None) == 4
    assert L.tree_weighted_nll(1, fake, fake, fake, 4, 8, -100, fake, None, None, fake, 1 << 20, None) == 5
    assert L.tree_weighted_nll(0, fake, fake, fake, 4, 8, -100, fake, None, None, None, 0, None) == 4
    assert L.tree_decode_splitkv(1, fake, fake, fake, fake, fake, 2, 4, 2, 64, 100, 0.0, 0, fake, fake, fake,
                                 1 << 20, None) == 5
    assert L.tree_decode_splitkv(1, fake, fake, fake, fake, fake, 2, 4, 2, 128, 100, 0.0, 0, fake, fake, None, 0,
                                 None) == 4
    n = ctypes.c_size_t()
    s = ctypes.c_int32()
    assert L.tree_decode_ws_bytes(8, 32, 128, 262144, 0, ctypes.byref(n), ctypes.byref(s)) == 0
    assert 1 <= s.value <= 120 and n.value >= 8 * 32 * s.value * 130 * 4
    assert L.tree_attn_ws_bytes(plan.handle, 3, 1, 4, 2, 128, 0.0, ctypes.byref(n)) == 1
    # the smallest backward workspace (op 2) is below the full one (op 1: plus the dS blocks)
    small, full = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.tree_attn_ws_bytes(plan.handle, 2, 1, 4, 2, 128, 0.0, ctypes.byref(small)) == 0
    assert L.tree_attn_ws_bytes(plan.handle, 1, 1, 4, 2, 128, 0.0, ctypes.byref(full)) == 0
    assert full.value >= small.value + plan.n_dsblk * 4 * 2048


def test_validation_before_launch_new_calls():
    """The output layer, partition and recurrent-layer calls also fail before
    any launch on arguments that are invalid on their face."""
    L = pkg.load_library()
    P = ctypes.c_void_p
    fake = P(0x1000)
    n = ctypes.c_size_t()
    # output layer: fp32 unsupported, Dm not a multiple of 32, dh without dW, workspace too small
    assert L.tree_lmhead_nll(0, fake, fake, fake, fake, 4, 100, 64, -100, 0, fake, None, None, None, None, fake,
                             1 << 30, None) == 5
    assert L.tree_lmhead_nll(1, fake, fake, fake, fake, 4, 100, 48, -100, 0, fake, None, None, None, None, fake,
                             1 << 30, None) == 5
    assert L.tree_lmhead_nll(1, fake, fake, fake, fake, 4, 100, 64, -100, 0, fake, None, fake, None, None, fake,
                             1 << 30, None) == 1
    assert L.tree_lmhead_nll(1, fake, fake, fake, fake, 4, 100, 64, -100, 0, fake, None, None, None, None, fake, 16,
                             None) == 4
    assert L.tree_lmhead_nll_ws_bytes(4, 100, 64, 1, 0, ctypes.byref(n)) == 0 and n.value > 0
    assert L.tree_lmhead_nll_ws_bytes(0, 100, 64, 1, 0, ctypes.byref(n)) == 1
    # partitioned attention: Hq not a multiple of Hkv; workspace too small
    part = pkg.tree_partition([-1, 0, 0], [40, 30, 30], 50)
    assert L.tree_partition_fwd(part.handle, fake, 1, fake, fake, fake, 3, 2, 128, 0.0, 0.0, fake, fake, fake,
                                1 << 30, None) == 1
    assert L.tree_partition_fwd(part.handle, fake, 1, fake, fake, fake, 4, 2, 128, 0.0, 0.0, fake, fake, fake, 16,
                                None) == 4
    assert L.tree_partition_ws_bytes(part.handle, 1, 1, 4, 2, 128, 0.0, ctypes.byref(n)) == 0 and n.value > 0
    # recurrent layers: null device tables, workspace too small, C <= 0
    plan = pkg.tree_plan([-1, 0], [300, 20])
    route = pkg.tree_route(plan, 4)
    assert L.tree_scan_fwd(route.handle, None, fake, fake, 8, fake, fake, 1 << 20, None) == 1
    assert L.tree_scan_fwd(route.handle, fake, fake, fake, 8, fake, fake, 16, None) == 4
    assert L.tree_scan_bwd(route.handle, fake, fake, fake, fake, 0, fake, fake, fake, 1 << 20, None) == 1
    assert L.tree_conv_bwd(route.handle, fake, fake, fake, fake, 8, fake, fake, fake, 16, None) == 4
    assert L.tree_scan_ws_bytes(route.handle, 8, ctypes.byref(n)) == 0 and n.value >= route.n_chunks * 8 * 4


def test_empty_plan_calls_touch_no_pointer():
    """A plan (or route) without tokens: the attention, scan and conv-forward
    calls return TA_OK after checking the plan, heads, d and dtype, before any
    tensor pointer is read, so empty tensors (null data pointers) are fine;
    invalid heads or d still fail first."""
    L = pkg.load_library()
    P = ctypes.c_void_p
    fake = P(0x1000)  # a device plan / route stand-in, never dereferenced
    plan = pkg.tree_plan([-1, 0], [0, 0])
    assert plan.n_tokens == 0
    assert L.tree_attn_fwd(plan.handle, fake, 1, None, None, None, 4, 2, 128, 0.0, 10000.0, None, None, None, 0,
                           None) == 0
    assert L.tree_attn_bwd(plan.handle, fake, 1, None, None, None, None, None, None, 4, 2, 128, 0.0, 10000.0,
                           None, None, None, None, 0, None) == 0
    assert L.tree_attn_fwd(plan.handle, fake, 1, None, None, None, 3, 2, 128, 0.0, 0.0, None, None, None, 0,
                           None) == 1
    assert L.tree_attn_bwd(plan.handle, fake, 1, None, None, None, None, None, None, 4, 2, 64, 0.0, 0.0,
                           None, None, None, None, 0, None) == 5
    route = pkg.tree_route(plan, 4)
    assert route.n_chunks == 0
    assert L.tree_scan_fwd(route.handle, fake, None, None, 8, None, None, 0, None) == 0
    assert L.tree_scan_bwd(route.handle, fake, None, None, None, 8, None, None, None, 0, None) == 0
    assert L.tree_conv_fwd(route.handle, fake, None, None, 8, None, None) == 0
    assert L.tree_scan_fwd(route.handle, fake, None, None, 0, None, None, 0, None) == 1
