"""Build of the HIP library libmsa_produce.so (gfx950) in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in ("msa_produce.hip", "msa_index.hip", "msa_unfused.hip", "msa_project.hip")]
LIB = os.path.join(PKG, "libmsa_produce.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: every multiply and add rounds on its own (no fused multiply-add);
# denormals are kept; binary32 division and square root are correctly rounded; packed-FP32
# instructions are switched off for the device code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    inc = os.path.join(ROOT, "include")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", inc, *SRCS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
