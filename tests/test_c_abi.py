"""include/gemm.h is a C header: a plain C99 program (tests/c_abi_check.c)
must compile against it with strict warnings, link libgemm.so and see the
documented host-side behaviour.  Runs without a GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

from tiled_gemm_f32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c_and_links():
    d = tempfile.mkdtemp(prefix="cabi_")
    try:
        exe = os.path.join(d, "cabi")
        lib_dir = os.path.dirname(_lib.LIB_PATH)
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Wpedantic", "-Werror",
               "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
               "-o", exe, "-L", lib_dir, "-lgemm", f"-Wl,-rpath,{lib_dir}"]
        build = subprocess.run(cmd, capture_output=True, text=True)
        assert build.returncode == 0, build.stderr
        out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout + out.stderr
    finally:
        shutil.rmtree(d, ignore_errors=True)
