"""The HIP sources compile for gfx950 with no kernel using scratch memory:
a spill or a dynamically indexed accumulator array would put the hot loops'
registers in private memory, which is correct but many times slower (an
unrolling failure in a GEMM epilogue once cost 4.6 ms per launch this way).
Runs hipcc on the host; no GPU."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from block_scaled_fp4_gather_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                                reason="hipcc not available")


def test_no_kernel_uses_scratch(tmp_path):
    procs = {}
    for src in build.SOURCES:
        out = tmp_path / (src + ".s")
        cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Rpass-analysis=kernel-resource-usage", "-o", str(out), os.path.join(build.CSRC, src)]
        procs[src] = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    bad = []
    kernels = 0
    for src, p in procs.items():
        text, _ = p.communicate(timeout=600)
        assert p.returncode == 0, text[-2000:]
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                kernels += 1
            m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
            if m and int(m.group(2)) != 0:
                bad.append(f"{src}: {name}: {m.group(1)} = {m.group(2)}")
    assert kernels >= 10
    assert not bad, "\n".join(bad)
