"""The library's host code (argument checks, sizing, layout arithmetic) under
AddressSanitizer: a build with the sanitizer on the host side only (device
code as usual) runs the host ABI tests in a child process with the ASan
runtime preloaded.  No GPU: every call those tests make returns before any
HIP launch."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from block_scaled_fp4_gather_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not RUNTIME or not os.path.exists(build.HIPCC), reason="no hipcc or no ASan runtime")
def test_host_code_under_asan(tmp_path):
    lib = tmp_path / "libmoe_fp4_asan.so"
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-o", str(lib)] + [os.path.join(build.CSRC, s) for s in build.SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-2000:]
    runner = (
        "import sys; sys.path.insert(0, %r)\n"
        "from block_scaled_fp4_gather_amd import moe\n"
        "moe.LIB_PATH = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, str(lib), os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=RUNTIME[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    run = subprocess.run([sys.executable, "-c", runner], capture_output=True, text=True, timeout=600, env=env,
                         cwd=ROOT)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "passed" in run.stdout and "AddressSanitizer" not in run.stderr
