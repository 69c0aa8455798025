"""Build the CPU oracle shared library (test infrastructure only).

Compiles ``oracle/gemv_ref.c`` and ``oracle/gla_ref.c`` with the host C compiler into
``oracle/libgemv_ref.so``.  Plain ``-O2`` with IEEE semantics kept
(``-fno-fast-math``, no FMA contraction), single-threaded code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemv_ref.c")
SRCS = [SRC, os.path.join(HERE, "gla_ref.c")]
LIB = os.path.join(HERE, "libgemv_ref.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall",
           "-Wextra", "-shared", "-fPIC"] + SRCS + ["-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
