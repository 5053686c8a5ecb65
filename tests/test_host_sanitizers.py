"""Host code under the address and undefined-behaviour sanitizers (CPU only).

- The oracle (oracle/svref.c) is compiled with gcc and both sanitizers into
  tests/sanitize/oracle_fuzz.c, which calls every oracle entry point on
  thousands of small random problems with every output and diagnostic
  requested and the awkward inputs the entry points promise to handle.
- The library's host side is compiled from the same sources as the product
  library (its device code unchanged and unsanitized) and linked into
  tests/sanitize/abi_checks.c, which drives every pure-host entry point and
  every launching entry point's argument checks with valid and mutated
  argument blocks (no GPU is touched).

A sanitizer report (out-of-bounds access, use after free, leak in the oracle,
signed overflow, invalid enum or shift) fails the test with the report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    run(["gcc", "-O1", "-g", "-std=gnu11", "-pthread", "-ffp-contract=off",
         "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "oracle"),
         os.path.join(SAN, "oracle_fuzz.c"), os.path.join(ROOT, "oracle", "svref.c"),
         "-o", exe, "-lm"])
    r = run([exe, "3000"], env=ENV, timeout=300)
    assert "oracle fuzz ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not available")
def test_library_host_side_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "rejection_sampling_verify_11_amd", "csrc")
    srcs = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    # device code as in the product build; the sanitizers on the host pass only
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
             "-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(f):
        obj = str(tmp_path / (f + ".o"))
        run([HIPCC, *flags, "-c", os.path.join(csrc, f), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_checks.o")
    run([CLANG, "-x", "c", "-std=c11", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
         "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
         "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-c",
         os.path.join(SAN, "abi_checks.c"), "-o", drv])
    exe = str(tmp_path / "abi_checks")
    run([CLANG + "++", "-fsanitize=address,undefined", drv, *objs,
         "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # the HIP runtime is not instrumented and keeps allocations to the end
    env = dict(ENV, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0")
    r = run([exe], env=env, timeout=300)
    assert "host checks ok" in r.stdout
