"""Builds libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_aux.hip"),
           os.path.join(CSRC, "kda_bwd.hip"), os.path.join(CSRC, "kda_noalloc.hip"),
           os.path.join(CSRC, "kda_generic.hip"),
           os.path.join(CSRC, "kda_api.cpp")]

# Device flags: gfx950 only; packed-fp32 instructions are turned off (the
# compiler still emits ordinary fp32 VALU code for the same arithmetic).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libkda.so)")


def build(resource_usage: bool = False) -> str:
    """Compile every source into gated_delta_rule_30_amd/libkda.so; always rebuilds."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkda.so")
    if resource_usage:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="-v" in sys.argv)
    print(LIB)
