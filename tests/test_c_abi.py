"""The C ABI from C: tests/c/abi_from_c.c, compiled as C99 with warnings as errors against
include/gsmi.h and linked against the built libgsmi.so, runs without a GPU (every call it makes
is refused by host validation or is a host-side query)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_DIR = os.path.join(ROOT, "differentiable_raster_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c_and_the_library_links():
    lib = os.path.join(LIB_DIR, "libgsmi.so")
    if not os.path.exists(lib):
        pytest.fail("libgsmi.so is not built (run __graft_entry__.build())")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "abi_from_c")
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
               os.path.join(HERE, "c", "abi_from_c.c"), "-L", LIB_DIR, "-lgsmi", f"-Wl,-rpath,{LIB_DIR}",
               "-Wl,--allow-shlib-undefined", "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "0 failure(s)" in r.stdout
