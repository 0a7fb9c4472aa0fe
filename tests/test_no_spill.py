"""Every kernel in the library compiles for gfx950 without spilling registers to scratch memory: a spill
puts per-lane stores and reloads on the memory path these kernels are bound by.  Reads the compiler's
resource-usage report for the device half of each source, with the library's own flags."""
import os
import re
import subprocess

import pytest

from paged_kv_cache_msa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _resource_usage(src):
    flags = [f for f in _build.HIP_FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    cmd = [_build.HIPCC, *flags, "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"), src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\d+) \[", line)
        if m and name is not None:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", _build.SRCS, ids=[os.path.basename(s) for s in _build.SRCS])
def test_kernels_do_not_spill(src):
    kernels = _resource_usage(src)
    assert kernels, "no kernels reported"
    spills = {k: v for k, v in kernels.items() if v.get("ScratchSize [bytes/lane]", -1) != 0}
    assert not spills, spills
