"""Builds tests/c_abi/verify_from_c: a plain C program (gcc, no HIP device
code) that calls libspecverify.so through include/specverify.h and checks it
against the CPU oracle compiled into it.  Test infrastructure; the GPU test
tests/test_gpu_c_abi.py runs the binary."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "rejection_sampling_verify_11_amd")
EXE = os.path.join(HERE, "verify_from_c")
ROCM = "/opt/rocm"


def build(exe: str = EXE) -> str:
    tmp = exe + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "oracle"),
           "-I" + os.path.join(ROCM, "include"),
           os.path.join(HERE, "verify_from_c.c"), os.path.join(ROOT, "oracle", "svref.c"),
           "-ffp-contract=off", "-o", tmp,
           "-L" + PKG, "-lspecverify", "-Wl,-rpath," + PKG,
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lm", "-pthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, exe)
    return exe


if __name__ == "__main__":
    print(build())
    sys.exit(0)
