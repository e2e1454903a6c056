"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain C, gcc, -O2 with IEEE semantics kept: no fused multiply-add contraction
and no fast-math, so every binary32 operation is rounded once, as written.
OpenMP only spreads independent output rows over threads; no result depends
on the thread count.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "p3d_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-fopenmp",
          "-Wall", "-Wextra", "-Werror"]


def build(src=SRC, out=LIB, extra=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
