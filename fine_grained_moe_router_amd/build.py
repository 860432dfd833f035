"""Build libmoedecode.so (gfx950) in-tree with hipcc.

    python -m fine_grained_moe_router_amd.build

The library is the C ABI declared in include/moe_decode.h: api.cpp (host-side
validation) and kernels.hip (gfx950 kernels). Packed-fp32 instruction selection is
disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoedecode.so")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "kernels.hip", "step.hip", "sample.hip", "draft.hip", "draft_fused.hip", "attn.hip")]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I" + INCLUDE, "-I" + CSRC, *DEVICE_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str, source: str = "kernels.hip") -> str:
    """Write the gfx950 assembly of one source file to out_path (for inspection)."""
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-I" + INCLUDE, "-I" + CSRC, *DEVICE_FLAGS, os.path.join(CSRC, source),
           "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
