"""The library driven by a plain C program through include/specverify.h
(tests/c_abi/verify_from_c.c): no Python or torch in that process, device
memory from the HIP runtime.  It runs one sampled verification, one greedy
verification and one KV rollback on seeded inputs and compares each with the
CPU oracle compiled into it (sampled outputs exact outside the oracle's
rounding bands, greedy and rollback bit-exact).  The GPU test runs the
program built by __graft_entry__.build() as a child process."""
import importlib.util
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("c_abi_build",
                                               os.path.join(HERE, "c_abi", "build.py"))
c_abi_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(c_abi_build)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_builds(tmp_path):
    exe = c_abi_build.build(str(tmp_path / "verify_from_c"))
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_c_program_through_the_abi():
    exe = c_abi_build.EXE
    assert os.path.exists(exe), "tests/c_abi/verify_from_c is not built: run __graft_entry__.build()"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi ok" in r.stdout
