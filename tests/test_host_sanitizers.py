"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_checks.cpp drives every entry point with invalid and
extreme arguments (null and misaligned pointers, negative and huge sizes,
unknown dtypes and status codes, too-small workspaces) and every size query
over a grid of extreme sizes, checking the status codes. It is linked with
the library's sources, the sanitizers on the host code only (each
-fsanitize= behind -Xarch_host; the kernels are built as usual). No GPU is
needed: every call is rejected by its argument checks before anything is
launched. A sanitizer report (an out-of-bounds host access, a signed
overflow in a size computation, an invalid enum value...) fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verification_sv_amd", "csrc")
SOURCES = ["sv_api.hip", "sv_chain.hip", "sv_lm_head.hip", "sv_sample.hip", "sv_tree.hip", "sv_tree_sample.hip"]


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is not installed")
def test_abi_checks_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-o", exe,
           os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), *[os.path.join(CSRC, s) for s in SOURCES]]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    print(run.stdout[-2000:], run.stderr[-4000:])
    assert run.returncode == 0, run.stderr[-4000:]
    assert " 0 failed" in run.stdout
