"""Build the gfx950 shared libraries with hipcc.

* ``_lib/liblittlebit.so`` -- the layer (include/littlebit.h): packing,
  decode and prefill kernels, the C ABI.  Links only the HIP runtime.
* ``_lib/liblittlebit_init.so`` -- the offline Dual-SVID initialization
  (include/littlebit_init.h).  Links rocBLAS and rocSOLVER; the layer
  library does not depend on it.

Usage: ``python -m binary_rank_gemv_amd.build`` (or ``build_library()``);
``--phase-stamps`` also builds ``_lib/stamped/liblittlebit.so``, the layer
library with phase timestamps in the one-token decode kernels.
Every call compiles from source (one hipcc process per source file, in
parallel, then one link per library); nothing is cached.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
OBJDIR = os.path.join(LIBDIR, "obj")
LIB = os.path.join(LIBDIR, "liblittlebit.so")
INIT_LIB = os.path.join(LIBDIR, "liblittlebit_init.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
# -amdgpu-kernarg-preload-count: the dispatch preloads up to 14 leading
# kernel-argument dwords into scalar registers (the decode kernel puts its
# phase-A fields there).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=14"]

LAYER_SOURCES = ("decode.hip", "decode1.hip", "littlebit_host.hip", "pack.hip", "prefill.hip")
INIT_SOURCES = ("init.hip",)


def sources():
    return [os.path.join(CSRC, f) for f in LAYER_SOURCES + INIT_SOURCES]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def _compile(src, verbose, extra_flags):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-c",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, *extra_flags,
          src, "-o", obj], verbose)
    return obj


def _link(objs, out, libs, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-L/opt/rocm/lib", *libs,
          "-Wl,-rpath,/opt/rocm/lib", "-o", tmp], verbose)
    os.replace(tmp, out)


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the CPU tests
# of the C ABI (device code is built as usual).
SANITIZE_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
SANITIZED_LIB = os.path.join(LIBDIR, "sanitized", "liblittlebit.so")


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload)."""
    out = subprocess.run([HIPCC.replace("hipcc", "amdclang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        out = found[-1] if found else ""
    return out


def build_sanitized_host(verbose: bool = False) -> str:
    """The layer library with its host-side C ABI code (littlebit_host.hip)
    built under ASan and UBSan, linked with the regular objects of the other
    sources (build_library must have run).  Load it with
    LITTLEBIT_LIBRARY=<path> and the ASan runtime preloaded."""
    objdir = os.path.join(LIBDIR, "sanitized")
    os.makedirs(objdir, exist_ok=True)
    host = os.path.join(objdir, "littlebit_host.hip.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-c",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, *SANITIZE_HOST_FLAGS,
          "-Xarch_host", "-fno-omit-frame-pointer", os.path.join(CSRC, "littlebit_host.hip"), "-o", host], verbose)
    others = [os.path.join(OBJDIR, f + ".o") for f in LAYER_SOURCES if f != "littlebit_host.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first; missing {missing}")
    _link([host, *others], SANITIZED_LIB, [*SANITIZE_HOST_FLAGS, "-shared-libsan"], verbose)
    return SANITIZED_LIB


STAMPED_LIB = os.path.join(LIBDIR, "stamped", "liblittlebit.so")


def build_phase_stamped(verbose: bool = False) -> str:
    """The layer library with phase timestamps in the decode kernels
    (decode1.hip and decode.hip built with -DLB_PHASE_STAMPS; they also
    export littlebit_phase_stamps_set and littlebit_phase_stamps_multi_set),
    linked with the regular objects of the other sources (build_library must
    have run).  For phase_timeline.py only."""
    objdir = os.path.join(LIBDIR, "stamped")
    os.makedirs(objdir, exist_ok=True)
    stamped = ("decode1.hip", "decode.hip")
    objs = []
    for f in stamped:
        obj = os.path.join(objdir, f + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-c", "-DLB_PHASE_STAMPS",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *DEVICE_FLAGS, os.path.join(CSRC, f), "-o", obj],
             verbose)
        objs.append(obj)
    others = [os.path.join(OBJDIR, f + ".o") for f in LAYER_SOURCES if f not in stamped]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first; missing {missing}")
    _link([*objs, *others], STAMPED_LIB, [], verbose)
    return STAMPED_LIB


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile both libraries; returns the layer library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip((os.path.basename(s) for s in srcs),
                        ex.map(lambda s: _compile(s, verbose, extra_flags), srcs)))
    _link([objs[f] for f in LAYER_SOURCES], LIB, [], verbose)
    _link([objs[f] for f in INIT_SOURCES], INIT_LIB, ["-lrocblas", "-lrocsolver"], verbose)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    if "--phase-stamps" in sys.argv:
        print(build_phase_stamped(verbose="-v" in sys.argv))
