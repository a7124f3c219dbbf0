"""Compiler resource report of the HIP kernels (hipcc cross-compiles for gfx950, no GPU needed):
no kernel keeps private arrays or spills in scratch memory, which would put a memory round trip
inside its loops."""
import re
import shutil
import subprocess

import pytest

from expert_offloaded_routed_amd import _build


def test_no_kernel_uses_scratch(tmp_path):
    try:
        hipcc = _build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if shutil.which(hipcc) is None and not hipcc.startswith("/"):
        pytest.skip("hipcc not available")
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
           "-I", _build.INCLUDE, "-I", _build.CSRC, *_build.DEVICE_FLAGS, "--cuda-device-only", "-c",
           f"{_build.CSRC}/moe_kernels.hip", "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    name, kernels, scratch = None, 0, []
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels += 1
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            scratch.append((name, int(m.group(1))))
    assert kernels > 0
    assert scratch == []
