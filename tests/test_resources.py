"""Register budget of every kernel, from the compiler's resource remarks
(CPU only: reads the last build's figures, or compiles the device code of
any source changed since).

The accumulator tiles live in registers only while every index into them is
known at compile time and the whole working set fits the register file;
otherwise the compiler moves them to per-lane scratch memory, a memory round
trip on every access of the hot loop ("Tiled matrix multiplication",
"Implementation notes" and "Pitfalls": check the build for spills).  So no
kernel may use scratch memory or spill vector registers, and the large-tile
ring kernels must keep their one-workgroup-per-CU register budget.
"""
import pytest

from tiled_gemm_f32_amd import build as hip_build


@pytest.fixture(scope="module")
def table():
    return hip_build.resource_usage()


def test_every_kernel_source_is_reported(table):
    import os
    sources = {k["source"] for k in table.values()}
    with_kernels = {s for s in hip_build.SOURCES
                    if s.endswith(".hip") and "__global__" in open(os.path.join(hip_build.CSRC, s)).read()}
    assert sources == with_kernels
    assert len(table) >= 60


def test_no_kernel_uses_scratch_or_spills_vector_registers(table):
    # Scalar registers spilled into lanes of a vector register (v_writelane)
    # stay in registers; only spills that reach scratch memory, and vector
    # register spills (which always do), count here.
    bad = [(k["name"], k.get("scratch"), k.get("vgpr_spill")) for k in table.values()
           if k.get("scratch", 1) != 0 or k.get("vgpr_spill", 1) != 0]
    assert not bad, "kernels with scratch memory or vector-register spills:\n" + "\n".join(map(str, bad))


def test_ring_kernels_fit_their_budget(table):
    rings = [k for k in table.values() if "ring_kernel" in k["name"] or "lines_kernel" in k["name"]]
    assert len(rings) >= 20
    for k in rings:
        # 256 architectural + 256 accumulation registers at most per lane, LDS within the 160 KB of a CU.
        assert k["vgprs"] <= 256 and k["agprs"] <= 256, k
        assert k["lds"] <= 160 * 1024, k
