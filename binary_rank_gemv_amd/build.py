"""Build the gfx950 shared library ``_lib/liblittlebit.so`` with hipcc.

Usage: ``python -m binary_rank_gemv_amd.build`` (or ``build_library()``).
Every call compiles from source; nothing is cached.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "liblittlebit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
# -amdgpu-kernarg-preload-count: the dispatch preloads up to 14 leading
# kernel-argument dwords into scalar registers (the decode kernel puts its
# phase-A fields there).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=14"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, *extra_flags,
           *sources(), "-L/opt/rocm/lib", "-lrocblas", "-lrocsolver", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
