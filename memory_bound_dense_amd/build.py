"""Build libgemv.so, the gfx950 GEMV library, in-tree.

    python -m memory_bound_dense_amd.build [-v]

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
turned off for the device code (-packed-fp32-ops).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemv.so")
SOURCES = [os.path.join(CSRC, "gemv.hip"), os.path.join(CSRC, "gla.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in ("gemv_kernel.h", "gemv_shift.h", "gemv_staged.h", "gla_kernel.h",
                                                     "handle.h")] + \
    [os.path.join(INCLUDE, "gemv.h"), os.path.join(INCLUDE, "gla_decode.h")]
# measurement aid: a plain streaming read (the practical HBM read ceiling)
PROBE_LIB = os.path.join(PKG, "libmbd_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _hipcc_shared(sources, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # the first 16 dwords of kernel arguments arrive in SGPRs at wave launch
           "-mllvm", "-amdgpu-kernarg-preload-count=16",
           "-I", INCLUDE, "-I", CSRC] + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc_shared(SOURCES, LIB, verbose)
    _hipcc_shared(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
