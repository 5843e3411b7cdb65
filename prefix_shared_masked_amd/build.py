"""Build the HIP library (gfx950) in-tree: prefix_shared_masked_amd/libtree_attn.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtree_attn.so")
SOURCES = ["plan.cpp", "partition.cpp", "gateway.hip", "attn_fwd.hip", "attn_bwd.hip", "nll.hip", "decode.hip",
           "lmhead.hip", "route.cpp", "ssm.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in arch VGPRs: the softmax reads them with VALU
    # ops, and the AGPR form made the register allocator copy the
    # loop-carried accumulators in and out of AGPRs every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wno-unused-command-line-argument",
]


def build_library(verbose: bool = False, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


# Host planner sources (plain C++, no device code): the tables the kernels read.
HOST_SOURCES = ["plan.cpp", "partition.cpp", "route.cpp"]


def build_host_sanitized(out_path: str) -> str:
    """The host planner alone (plan, partition, route) built with g++ under
    AddressSanitizer and UndefinedBehaviorSanitizer, as a shared library the
    binding can load in host-only mode (for the sanitized planner test)."""
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stderr}")
    return out_path


if __name__ == "__main__":
    print(build_library(verbose=True))
