"""Builds the CPU oracle library (oracle/libsvref.so) with gcc.

Test infrastructure: the oracle is compiled as plain C11 + pthreads, with no
fast-math and no floating-point contraction, so its arithmetic is strict IEEE
fp64.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "svref.c")
LIB = os.path.join(HERE, "libsvref.so")
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
          "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(
            os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "svref.h"))):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
