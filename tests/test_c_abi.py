"""include/carve.h is usable from plain C: a C99 program that includes it compiles with
warnings as errors, links against the built library and passes its host-side checks
(CPU only: every call it makes is answered or rejected before any launch)."""
import os
import shutil
import subprocess

import pytest

from chunk_gated_delta_amd import carve

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c_and_library_links(tmp_path):
    lib = carve.LIB_PATH
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe), lib,
           "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "carve C ABI: ok" in r.stdout
