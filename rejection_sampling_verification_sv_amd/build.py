"""Build libspecverify.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m rejection_sampling_verification_sv_amd.build [--verbose]

hipcc cross-compiles without a GPU. The library lands next to this file,
where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["sv_api.hip", "sv_chain.hip", "sv_lm_head.hip", "sv_sample.hip", "sv_tree.hip", "sv_tree_sample.hip"]
HEADERS = ["sv_device.h", "sv_internal.h", "sv_stream.h"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep every floating-point contraction explicit (fmaf) so that repeated
    # evaluations of the same weights are bit-identical
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libspecverify)")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles). Returns the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(REPO_DIR, "include"), "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # the host pass warns that it does not know the packed-fp32 feature
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
