"""Build libqgemv.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU instructions are disabled for all device code. Matrix-core
# results go straight to VGPRs (the small-N kernel scales every product in fp32;
# AGPR results would cost one copy instruction per element).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = True, resource_report: str | None = None) -> str:
    """Compile every .hip source into one shared library. If resource_report is a
    path, the compiler's per-kernel resource usage (VGPRs, SGPRs, scratch, LDS,
    occupancy) is written there."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources()]
    if resource_report:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    # the host pass does not know the device-only feature name; that note is harmless
    noise = "is not a recognized feature for this target"
    text = "\n".join(l for l in out.splitlines() if noise not in l)
    if resource_report:
        with open(resource_report, "w") as f:
            f.write(text + "\n")
    if res.returncode != 0:
        sys.stderr.write(text + "\n")
        raise RuntimeError("hipcc failed with status %d" % res.returncode)
    if verbose and text.strip() and not resource_report:
        print(text)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    rep = sys.argv[1] if len(sys.argv) > 1 else None
    print(build(resource_report=rep))
