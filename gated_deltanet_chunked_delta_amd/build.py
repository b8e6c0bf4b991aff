"""Builds libgdn.so (the C-ABI library of include/gdn.h) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree and is the one the Python binding loads.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = [os.path.join(PKG, "csrc", "gdn_fused.hip"), os.path.join(PKG, "csrc", "gdn_fused_ws.hip"),
           os.path.join(PKG, "csrc", "gdn_recurrent.hip"), os.path.join(PKG, "csrc", "gdn_gating.hip"),
           os.path.join(PKG, "csrc", "gdn_split.hip"), os.path.join(PKG, "csrc", "gdn_backward.hip"),
           os.path.join(PKG, "csrc", "gdn_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "gdn.h"), os.path.join(PKG, "csrc", "gdn_internal.h"),
           os.path.join(PKG, "csrc", "gdn_device.h")]

# Packed fp32 VALU instructions are kept out of the generated code.  MFMA
# accumulators are kept in VGPRs: the kernels consume every accumulator with
# VALU code, and the AGPR form costs a copy in and out of each product.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
