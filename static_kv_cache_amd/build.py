"""Build libkvc.so in-tree with hipcc for gfx950.

The library is one shared object compiled from ``csrc/*.hip`` against the
public header ``include/kvc.h``. Packed fp32 instructions are disabled
(``-packed-fp32-ops``; the host pass warns that it does not know that
feature, which is harmless). MFMA accumulators are kept in ordinary VGPRs
(``-amdgpu-mfma-vgpr-form``), so the softmax rescale works on them in place
instead of copying them out of and back into AGPRs.
"""

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-mcode-object-version=5", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build_library(verbose=False):
    """Compile every HIP source into libkvc.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msg}")
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
