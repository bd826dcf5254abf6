"""The workgroup -> tile mapping (XCD regrouping + banded order) must be a
bijection onto the tile grid; checked on the host by compiling the same
device header as host code."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_tile_mapping_is_a_bijection():
    d = tempfile.mkdtemp(prefix="tilemap_")
    try:
        exe = os.path.join(d, "check")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
                        "-I", os.path.join(ROOT, "tiled_gemm_f32_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "tile_map_check.cpp"), "-o", exe],
                       check=True, capture_output=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0, out.stdout
        assert out.stdout.startswith("OK")
    finally:
        shutil.rmtree(d, ignore_errors=True)
