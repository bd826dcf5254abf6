"""The C ABI on the host: exported symbols, argument validation and kernel
choice.  Nothing here launches GPU work; validation and planning are plain
host code, so they run (and are tested) without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")

F32, BF16, FP8 = tg.GEMM_DTYPE_F32, tg.GEMM_DTYPE_BF16F32, tg.GEMM_DTYPE_FP8F32
N_, T_ = tg.GEMM_OP_N, tg.GEMM_OP_T
OK, INVALID, UNSUP = tg.GEMM_OK, tg.GEMM_ERR_INVALID_ARG, tg.GEMM_ERR_UNSUPPORTED
# Fake but well-aligned device addresses: planning only inspects them.
PA, PB, PC = 0x7f0000000000, 0x7f1000000000, 0x7f2000000000


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"GEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def plan(dtype, M, N, K, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, beta=0.0, C=PC, ldc=None, force=0, ws=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return tg.gemm_plan_query(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force, ws)


def kernel_ids(**match):
    return [k["id"] for k in tg.kernels() if all(k[f] == v for f, v in match.items())]


# ----------------------------------------------------------------------------- library

def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    # Hidden visibility: nothing but the ABI (and runtime glue) leaks out.
    assert not [s for s in exported if "gemm" in s and s not in names]


def test_status_strings():
    for st in range(6):
        s = tg.gemm_status_string(st)
        assert s and s != "unknown status"
    assert tg.gemm_status_string(99) == "unknown status"


def test_kernel_table_is_consistent():
    ks = tg.kernels()
    assert len(ks) == tg.gemm_kernel_count() > 0
    assert [k["id"] for k in ks] == list(range(1, len(ks) + 1))
    assert len({k["name"] for k in ks}) == len(ks)
    for k in ks:
        assert k["dtype"] in (F32, BF16, FP8)
        assert k["path"] in (tg.GEMM_PATH_TILED, tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK)
        assert 1 <= k["layouts"] <= 15
        assert k["threads"] % 64 == 0 and 64 <= k["threads"] <= 1024
        if k["path"] == tg.GEMM_PATH_TILED:
            assert k["tile_m"] % 32 == 0 and k["tile_n"] % 32 == 0
    with pytest.raises(tg.GemmError):
        tg.gemm_kernel_query(0)
    with pytest.raises(tg.GemmError):
        tg.gemm_kernel_query(len(ks) + 1)


# ----------------------------------------------------------------------------- validation

@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("kwargs", [
    dict(M=-1, N=4, K=4), dict(M=4, N=-1, K=4), dict(M=4, N=4, K=-1),
    dict(M=4, N=4, K=8, lda=7), dict(M=4, N=8, K=4, ldb=7), dict(M=4, N=8, K=4, ldc=7),
    dict(M=4, N=4, K=0, lda=0), dict(M=4, N=4, K=4, C=0), dict(M=4, N=4, K=4, A=0), dict(M=4, N=4, K=4, B=0),
    dict(M=4, N=4, K=4, C=PC + 2),
])
def test_invalid_arguments_rejected(dtype, kwargs):
    st, _ = plan(dtype, **kwargs)
    assert st == INVALID


def test_misaligned_element_pointers_rejected():
    assert plan(F32, 4, 4, 4, A=PA + 2)[0] == INVALID
    assert plan(BF16, 4, 4, 4, A=PA + 1)[0] == INVALID
    assert plan(BF16, 4, 4, 4, A=PA + 2)[0] == OK       # 2-byte aligned is enough for bf16


def test_operands_not_needed_may_be_null():
    assert plan(F32, 4, 4, 0, A=0, B=0)[0] == OK        # K == 0: A, B not read
    assert plan(F32, 4, 4, 4, alpha=0.0, A=0, B=0)[0] == OK
    assert plan(F32, 0, 4, 4, A=0, B=0, C=0)[0] == OK   # empty C


def test_unsupported_sizes():
    assert plan(F32, 2 ** 31, 4, 4)[0] == UNSUP
    assert plan(F32, 4, 4, 4, lda=2 ** 31)[0] == UNSUP
    assert plan(F32, 4, 4, 4, ldb=2 ** 31)[0] == UNSUP
    assert plan(F32, 4, 4, 4, lda=2 ** 31 - 1)[0] == OK
    assert plan(F32, 4, 4, 4, ldb=2 ** 31 - 1)[0] == OK


def test_large_operands_keep_their_fast_kernels():
    """Buffer offsets are 32-bit per panel or slice, not per operand: weights
    of 2 GiB and more stay on the streaming kernels, and a leading dimension
    of 2^21 elements or more on the tiled ones, as long as one panel fits."""
    # 16 x 65536 x 8192 fp32 and 16 x 131072 x 8192 bf16: B is 2 GiB.
    st, pl = plan(F32, 16, 65536, 8192)
    assert st == OK and pl["path"] == tg.GEMM_PATH_SKINNY, kname(pl)
    st, pl = plan(F32, 16, 65536, 8192, ws=1 << 30)
    assert st == OK and pl["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK), kname(pl)
    st, pl = plan(BF16, 16, 131072, 8192)
    assert st == OK and pl["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK), kname(pl)
    st, pl = gplan(F32, T_, N_, 16, 65536, 8192, lda=16)
    assert st == OK and pl["path"] == tg.GEMM_PATH_SKINNY, kname(pl)
    # B with more than 2^21 columns (2.1 GB at K = 256): a ring kernel, whose
    # B slices are 16 rows deep.
    st, pl = plan(F32, 64, (1 << 21) + 64, 256)
    assert st == OK and "general" not in kname(pl) and pl["tile_k"] == 16, kname(pl)
    st, pl = plan(BF16, 512, (1 << 22) + 64, 256)
    assert st == OK and "general" not in kname(pl), kname(pl)
    # A with rows 2^22 floats apart: 256- and 128-row panels would span more
    # than 2^31 bytes, 64-row ones do not.
    st, pl = plan(F32, 1024, 1024, 4096, lda=1 << 22)
    assert st == OK and pl["tile_m"] == 64 and "general" not in kname(pl), kname(pl)
    # Too far apart for any panel: the general kernel (64-bit element offsets).
    st, pl = plan(F32, 1024, 1024, 4096, lda=1 << 25)
    assert st == OK and "general" in kname(pl), kname(pl)
    # A skinny call whose 16 rows of A span more than 2^31 bytes is not streamed.
    st, pl = plan(F32, 16, 8192, 4096, lda=1 << 26)
    assert st == OK and pl["path"] == tg.GEMM_PATH_TILED, kname(pl)


def test_invalid_dtype_and_force():
    assert plan(7, 4, 4, 4)[0] == INVALID
    assert plan(F32, 4, 4, 4, force=-1)[0] == INVALID
    assert plan(F32, 4, 4, 4, force=tg.gemm_kernel_count() + 1)[0] == INVALID


def test_argument_errors_return_before_any_device_call():
    # Invalid calls come back from the real entry points without a GPU.
    lib = _lib.load()
    assert tg.gemm_f32(-1, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, 0) == INVALID
    assert tg.gemm_bf16f32(4, 4, 8, 1.0, PA, 7, PB, 4, 0.0, PC, 4, 0) == INVALID
    assert tg.gemm_f32_ex(4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, -5, None, 0, 0, 0) == INVALID
    assert tg.gemm_f32_ws(4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, PC + 2, 64, 0) == INVALID   # misaligned ws
    assert tg.gemm_f32_ws(4, 4, 4, 1.0, PA, 4, PB, 4, 0.0, PC, 4, PC, -1, 0) == INVALID
    assert lib is not None


def test_epilogue_argument_errors():
    """An unknown activation or a bias not 4-byte aligned is rejected on the
    host; a NULL descriptor and a well-formed one are accepted (M == 0 is a
    no-op, so nothing reaches the device)."""
    for fn, a, b in ((tg.gemm_f32_epi, PA, PB), (tg.gemm_bf16f32_epi, PA, PB)):
        args = (4, 8, 8, 1.0, a, 8, b, 8, 0.0, PC, 8)
        for act in (-1, 3, 99):
            assert fn(*args, tg.Epilogue(None, act), 0, 0, 0) == INVALID, act
        assert fn(*args, tg.Epilogue(PC + 2, tg.GEMM_ACT_RELU), 0, 0, 0) == INVALID
        empty = (0,) + args[1:]
        assert fn(*empty, None, 0, 0, 0) == OK
        for act in (tg.GEMM_ACT_NONE, tg.GEMM_ACT_RELU, tg.GEMM_ACT_GELU):
            assert fn(*empty, tg.Epilogue(PC, act), 0, 0, 0) == OK
    assert tg.gemm_f32_ex(4, 8, 8, 1.0, PA, 8, PB, 8, 0.0, PC, 8, 0, tg.Epilogue(None, 5), 0, 0, 0) == INVALID
    assert tg.gemm_bf16f32_ex(4, 8, 8, 1.0, PA, 8, PB, 8, 0.0, PC, 8, 0, (PC + 1, 0), 0, 0, 0) == INVALID


def test_activation_codes_match_header():
    with open(HEADER) as f:
        text = f.read()
    for name in ("GEMM_ACT_NONE", "GEMM_ACT_RELU", "GEMM_ACT_GELU"):
        m = re.search(rf"{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(tg, name), name


# ----------------------------------------------------------------------------- quick returns

def test_quick_return_paths():
    assert plan(F32, 0, 10, 10)[1]["path"] == tg.GEMM_PATH_NONE
    assert plan(F32, 10, 0, 10)[1]["path"] == tg.GEMM_PATH_NONE
    st, p = plan(F32, 10, 10, 0)
    assert st == OK and p["path"] == tg.GEMM_PATH_SCALE and p["kernel_id"] == 0
    assert plan(BF16, 10, 10, 10, alpha=0.0)[1]["path"] == tg.GEMM_PATH_SCALE


# ----------------------------------------------------------------------------- kernel choice

def test_skinny_path_for_m_up_to_16():
    for M in (1, 7, 16):
        st, p = plan(F32, M, 8192, 8192)
        assert st == OK and p["path"] == tg.GEMM_PATH_SKINNY and p["tile_m"] == 16
    st, p = plan(F32, 17, 8192, 8192)
    assert p["path"] == tg.GEMM_PATH_TILED
    # bf16 without a workspace: its streaming kernel over the whole of K.
    assert plan(BF16, 16, 8192, 8192)[1]["path"] == tg.GEMM_PATH_SKINNY
    assert plan(BF16, 17, 8192, 8192)[1]["path"] == tg.GEMM_PATH_TILED


def test_skinny_decode_shape_fills_the_chip():
    st, p = plan(F32, 16, 8192, 8192)
    assert p["grid"] == 256 and p["vec_b"] == 2 and p["tile_n"] == 32


def test_skinny_streams_any_size_and_falls_back_only_when_a_batch_overflows():
    # 16 GiB of B: the streaming kernels rebase B per batch of k rows.
    st, p = plan(F32, 16, 65536, 65536)
    assert st == OK and p["path"] == tg.GEMM_PATH_SKINNY
    # One batch of 512 rows of 2^21 floats spans 4 GiB: not streamed by those.
    st, p = plan(F32, 16, 1 << 21, 4096)
    assert st == OK and kname(p) != "f32_skinny_mfma16_n2_a4_w8_u4", kname(p)


@pytest.mark.parametrize("M,N,K,tile,grid", [
    (4096, 4096, 4096, 256, 256), (4092, 4092, 4092, 256, 256), (256, 256, 256, 64, 16),
    (1000, 3000, 777, 64, 16 * 47)])
def test_f32_tile_choice(M, N, K, tile, grid):
    st, p = plan(F32, M, N, K)
    assert st == OK and p["path"] == tg.GEMM_PATH_TILED
    assert (p["tile_m"], p["grid"]) == (tile, grid)
    # A workspace changes the choice only where it buys a K split (or a
    # larger tile that still fills a whole wave).
    st, pw = plan(F32, M, N, K, ws=1 << 30)
    assert st == OK and (pw["splits"] > 1 or pw["grid"] >= 256 or (pw["tile_m"], pw["grid"]) == (tile, grid)), pw
    if (M, N, K) == (1000, 3000, 777):
        assert (pw["tile_m"], pw["splits"]) == (64, 1), pw


def test_bf16_tile_choice():
    st, p = plan(BF16, 8192, 8192, 8192)
    assert (p["tile_m"], p["tile_n"], p["grid"], p["vec_a"], p["vec_b"]) == (256, 256, 1024, 8, 8)


def test_bf16_mid_size_choice():
    """bf16 (and fp8) problems with 256 to 1023 tiles of 128^2 take a 128 x
    128 whole-line kernel; with a workspace it is still preferred, unsplit,
    over 256^2 tiles split over K (the split's workspace round trip costs
    more than the smaller tile gives up), and fp32 takes its 128^2 ring the
    same way."""
    L128 = "bf16_mfma32_128x128x64_w2x2_a8b8_lines"
    for M, N, K in [(2048, 2048, 2048), (2048, 4096, 4096), (2048, 2048, 8192), (1536, 1536, 4096)]:
        for ws in (0, 1 << 34):
            st, p = plan(BF16, M, N, K, ws=ws)
            assert st == OK and kname(p) == L128 and p["splits"] == 1, (M, N, K, ws, p)
    st, p = plan(BF16, 4096, 4096, 4096, ws=1 << 34)
    assert kname(p) == "bf16_mfma32_256x256x64_w2x2_a8b8_lines" and p["splits"] == 1
    # Too few 128^2 tiles to fill the compute units: the split 256^2 tiles.
    st, p = plan(BF16, 1024, 1024, 16384, ws=1 << 34)
    assert p["tile_m"] == 256 and p["splits"] == 16, p
    # fp32 likewise, on the 128^2 ring.
    st, p = plan(F32, 2048, 4096, 4096, ws=1 << 34)
    assert kname(p) == "f32_mfma32_128x128x16_w2x2_a4b4_ring4" and p["splits"] == 1, p
    # B stored N x K (a linear layer's weights) and A stored K x M (its
    # weight gradient): the same choice in those layouts.
    for M, N, K in [(2048, 2048, 2048), (2048, 4096, 4096)]:
        for ws in (0, 1 << 34):
            st, p = gplan(BF16, N_, T_, M, N, K, ws=ws)
            assert st == OK and kname(p) == "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines" and p["splits"] == 1, p
            st, p = gplan(BF16, T_, N_, M, N, K, ws=ws)
            assert st == OK and kname(p) == "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines" and p["splits"] == 1, p
    # fp8 with B stored N x K likewise.
    for ws in (0, 1 << 34):
        st, p = gplan(FP8, N_, T_, 2048, 4096, 4096, ws=ws)
        assert st == OK and kname(p) == "fp8_mfma32_128x128x128_w2x2_nt_lines" and p["splits"] == 1, p
    # Below its minimum K the generic 128^2 kernel runs.
    st, p = plan(BF16, 2048, 2048, 128)
    assert st == OK and p["tile_m"] == 128 and kname(p) != L128, p


def test_vector_width_follows_alignment():
    # K = 777: rows of A are not 16-byte aligned -> element loads for A only.
    st, p = plan(F32, 1000, 3000, 777)
    assert (p["vec_a"], p["vec_b"]) == (1, 4)
    # A base pointer off by 4 bytes.
    assert plan(F32, 4096, 4096, 4096, A=PA + 4)[1]["vec_a"] == 1
    # ldb not a multiple of 4.
    assert plan(F32, 4096, 4094, 4096, ldb=4094)[1]["vec_b"] == 1
    assert plan(BF16, 8192, 8192, 8188)[1]["vec_a"] == 1


def test_forced_kernels():
    nn = {k["id"] for k in tg.kernels() if k["layouts"] & 1}
    f32_tiled = [k for k in kernel_ids(dtype=F32, path=tg.GEMM_PATH_TILED) if k in nn]
    bf16_tiled = [k for k in kernel_ids(dtype=BF16, path=tg.GEMM_PATH_TILED) if k in nn]
    skinny = kernel_ids(dtype=F32, path=tg.GEMM_PATH_SKINNY, layouts=1)
    assert f32_tiled and bf16_tiled and skinny
    for kid in f32_tiled:
        st, p = plan(F32, 512, 512, 512, force=kid)
        assert st == OK and p["kernel_id"] == kid
        assert plan(BF16, 512, 512, 512, force=kid)[0] == UNSUP
    for kid in skinny:
        assert plan(F32, 16, 512, 512, force=kid)[0] == OK
        assert plan(F32, 17, 512, 512, force=kid)[0] == UNSUP
    # A 4-wide-A kernel cannot take K = 777.
    wide_a = [k for k in f32_tiled if tg.gemm_kernel_query(k)["vec_a"] == 4]
    assert all(plan(F32, 1000, 3000, 777, force=k)[0] == UNSUP for k in wide_a)
    # Workspace kernels need a workspace of the advertised size.
    split = kernel_ids(dtype=F32, path=tg.GEMM_PATH_SKINNY_SPLITK, layouts=1)
    assert split
    need = tg.gemm_workspace_size(F32, 16, 512, 4096)
    for kid in split:
        assert plan(F32, 16, 512, 4096, force=kid, ws=need)[0] == OK
        assert plan(F32, 16, 512, 4096, force=kid, ws=need - 4)[0] == UNSUP
        assert plan(F32, 16, 512, 4096, force=kid)[0] == UNSUP


# ----------------------------------------------------------------------------- workspace path

def test_workspace_size():
    MiB = 1 << 20
    # 16 x 8192 x 8192 fp32: the skinny split needs 4 slices x 16 x 8192 fp32 (2 MiB); the tiled
    # split of 32 tiles of 256 x 256 into 8 slices of 1024 needs 8 x 16 x 8192 fp32 (4 MiB).
    # The larger of the two is returned.
    assert tg.gemm_workspace_size(F32, 16, 8192, 8192) == 8 * 16 * 8192 * 4 == 4 * MiB
    assert tg.gemm_workspace_size(BF16, 16, 8192, 8192) == 8 * 16 * 8192 * 4
    assert tg.gemm_workspace_size(F32, 17, 8192, 8192) == 8 * 17 * 8192 * 4
    assert tg.gemm_workspace_size(F32, 16, 8192, 0) == 0
    # Skinny slices are at least 512 deep, tiled ones at least 1024: K = 1024 gives 2 skinny
    # slices and no tiled split; K = 1023 neither.
    assert tg.gemm_workspace_size(F32, 1, 256, 1024) == 2 * 1 * 256 * 4
    assert tg.gemm_workspace_size(F32, 1, 256, 1023) == 0
    # Partials hold M rows: 7 x 1000 with 8 strips and K = 4100 -> 8 skinny slices (the tiled
    # split of its 4 tiles would take 4 slices of 1088).
    assert tg.gemm_workspace_size(F32, 7, 1000, 4100) == 8 * 7 * 1000 * 4
    # Tiled split: 1024 x 1024 x 16384 has 16 tiles -> 16 slices of 1024.
    assert tg.gemm_workspace_size(F32, 1024, 1024, 16384) == 16 * 1024 * 1024 * 4
    assert tg.gemm_workspace_size(BF16, 1024, 1024, 16384) == 16 * 1024 * 1024 * 4
    # Enough tiles already (4096^3: 256 tiles): no split, no workspace.
    assert tg.gemm_workspace_size(F32, 4096, 4096, 4096) == 0
    assert tg.gemm_workspace_size(BF16, 8192, 8192, 8192) == 0
    assert tg.gemm_workspace_size(2, 16, 16, 16) == 0


def test_workspace_selects_split_k_for_decode_shape():
    need = tg.gemm_workspace_size(F32, 16, 8192, 8192)
    skinny_need = 4 * 16 * 8192 * 4
    st, p = plan(F32, 16, 8192, 8192, ws=need)
    assert st == OK and p["path"] == tg.GEMM_PATH_SKINNY_SPLITK and p["grid"] == 256 and p["tile_n"] == 128
    assert p["splits"] == 1
    assert plan(F32, 16, 8192, 8192, ws=skinny_need)[1]["path"] == tg.GEMM_PATH_SKINNY_SPLITK
    assert plan(F32, 16, 8192, 8192, ws=skinny_need - 1)[1]["path"] == tg.GEMM_PATH_SKINNY
    assert plan(F32, 16, 8192, 8192)[1]["path"] == tg.GEMM_PATH_SKINNY


def test_workspace_tiled_k_split_plan():
    """Few output tiles and a deep K: with a workspace the 256 x 256 kernel is
    split along K so that tiles x slices fills the compute units."""
    for dt in (F32, BF16):
        need = tg.gemm_workspace_size(dt, 1024, 1024, 16384)
        st, p = plan(dt, 1024, 1024, 16384, ws=need)
        assert st == OK and p["path"] == tg.GEMM_PATH_TILED and p["tile_m"] == 256
        assert p["splits"] == 16 and p["grid"] == 16 * 16
        # No workspace: smaller tiles, unsplit (fp32 has 64 x 64 kernels, 256 tiles; bf16's
        # smallest tile is 128 x 128, 64 tiles).  Too small a workspace for the 16-way
        # 256 x 256 split: the 128 x 128 kernel split 4 ways (16 MiB) fills the chip.
        st, p = plan(dt, 1024, 1024, 16384)
        assert st == OK and p["splits"] == 1
        assert (p["tile_m"], p["grid"]) == ((64, 256) if dt == F32 else (128, 64))
        st, p = plan(dt, 1024, 1024, 16384, ws=need - 4)
        assert st == OK and (p["tile_m"], p["splits"], p["grid"]) == (128, 4, 256)
        # 17 x 8192 x 8192 (not skinny): a 256-row tile would be 93% padding; no tile size
        # wastes under a quarter, so the usual choice (the smallest tile) is split instead.
        need = tg.gemm_workspace_size(dt, 17, 8192, 8192)
        st, p = plan(dt, 17, 8192, 8192, ws=need)
        assert st == OK
        assert (p["tile_m"], p["splits"], p["grid"]) == ((64, 2, 256) if dt == F32 else (128, 4, 256))
        # 100 x 4096 x 8192: 128-row tiles waste 22% -> 32 tiles x 8 slices.
        st, p = plan(dt, 100, 4096, 8192, ws=tg.gemm_workspace_size(dt, 100, 4096, 8192))
        assert st == OK and (p["tile_m"], p["splits"], p["grid"]) == (128, 8, 256)
    # A 256 x 256 split that would fill under three quarters of the compute units is not
    # preferred over smaller tiles: 512 x 1024 has 8 such tiles (8 x 16 = 128 workgroups);
    # the 128 x 128 kernel (32 tiles) split in 8 is taken instead.
    for dt, tile, splits in ((F32, 128, 8), (BF16, 128, 8)):
        need = tg.gemm_workspace_size(dt, 512, 1024, 16384)
        st, p = plan(dt, 512, 1024, 16384, ws=need)
        assert st == OK and (p["tile_m"], p["splits"], p["grid"]) == (tile, splits, 256)
    # Slices are whole multiples of 64 deep: 256 x 512 x 4100 on 64 x 64 tiles (32 tiles)
    # -> 4 slices of 1088 (the last one 836).
    st, p = plan(F32, 256, 512, 4100, ws=tg.gemm_workspace_size(F32, 256, 512, 4100))
    assert st == OK and p["tile_m"] == 64 and p["splits"] == 4 and p["grid"] == 128
    # No split where K is shallow or the problem already fills the chip.
    assert plan(F32, 1024, 1024, 1500, ws=1 << 30)[1]["splits"] == 1
    assert plan(F32, 4096, 4096, 4096, ws=1 << 30)[1]["splits"] == 1
    # Quick-return paths report no split.
    assert plan(F32, 0, 16, 16, ws=1 << 30)[1]["splits"] == 0
    assert plan(F32, 16, 16, 0, ws=1 << 30)[1]["splits"] == 0




# ----------------------------------------------------------------------------- tuning table

def _kid(name):
    return [k["id"] for k in tg.kernels() if k["name"] == name][0]


def test_tuning_table_load_save_and_plan(tmp_path):
    """A tuning table written as text steers the automatic choice for its key
    (dtype, shape, alignment class, workspace presence) and only that key."""
    tg.gemm_tuning_clear()
    assert tg.gemm_tuning_count() == 0
    f = tmp_path / "table.txt"
    f.write_text("# comment\n"
                 "0 1024 1024 1024 4 4 0 f32_mfma32_128x128x16_w2x2_a4b4 0 0.5\n"
                 "1 2048 2048 8192 8 8 1 bf16_mfma32_128x128x64_w2x2_a8b8 0 0.1\n"
                 "0 512 512 512 4 4 0 no_such_kernel 0 0.1\n")
    assert tg.gemm_tuning_load(str(f)) == 2          # the unknown kernel is skipped
    assert tg.gemm_tuning_count() == 2
    st, p = plan(F32, 1024, 1024, 1024)
    assert st == OK and p["kernel_id"] == _kid("f32_mfma32_128x128x16_w2x2_a4b4")
    # Another alignment class (A not 16-byte aligned) or shape: the built-in choice.
    assert plan(F32, 1024, 1024, 1024, A=PA + 4)[1]["kernel_id"] != _kid("f32_mfma32_128x128x16_w2x2_a4b4")
    assert plan(F32, 1024, 1024, 1032)[1]["kernel_id"] != _kid("f32_mfma32_128x128x16_w2x2_a4b4")
    # A recorded "no split" is honoured even with a workspace large enough for one.
    st, p = plan(BF16, 2048, 2048, 8192, ws=1 << 30)
    assert st == OK and p["kernel_id"] == _kid("bf16_mfma32_128x128x64_w2x2_a8b8") and p["splits"] == 1
    st, p = plan(BF16, 2048, 2048, 8192)              # no workspace: another key
    assert p["kernel_id"] != _kid("bf16_mfma32_128x128x64_w2x2_a8b8") or p["splits"] == 1
    # Forced kernels ignore the table.
    other = _kid("f32_mfma32_64x64x16_w2x2_a4b4")
    assert plan(F32, 1024, 1024, 1024, force=other)[1]["kernel_id"] == other
    # Save and reload round trip.
    out = tmp_path / "saved.txt"
    assert tg.gemm_tuning_save(str(out)) == OK
    lines = [l for l in out.read_text().splitlines() if not l.startswith("#")]
    assert out.read_text().startswith("# libgemm tuning table v2")
    assert len(lines) == 2 and all(len(l.split()) == 12 and l.split()[1:3] == ["0", "0"] for l in lines)
    tg.gemm_tuning_clear()
    assert tg.gemm_tuning_count() == 0
    assert tg.gemm_tuning_load(str(out)) == 2
    assert plan(F32, 1024, 1024, 1024)[1]["kernel_id"] == _kid("f32_mfma32_128x128x16_w2x2_a4b4")
    tg.gemm_tuning_clear()


def test_tuning_table_layouts(tmp_path):
    """Format v2 keys entries by layout as well: an entry for A x B^T steers
    gemm_general calls of that layout only; entries naming a kernel without
    that layout are skipped; op values other than N/T make the file invalid."""
    tg.gemm_tuning_clear()
    f = tmp_path / "v2.txt"
    f.write_text("# libgemm tuning table v2: dtype op_a op_b M N K vec_a vec_b has_ws kernel split ms\n"
                 "1 0 1 4096 4096 4096 8 8 0 bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4 0 0.2\n"
                 "2 1 0 2048 2048 2048 16 16 0 fp8_general_128x128x16 0 0.3\n"
                 "1 1 1 4096 4096 4096 8 8 0 bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4 0 0.2\n")
    assert tg.gemm_tuning_load(str(f)) == 2          # the NT ring cannot run T x T: skipped
    # Untuned built-in choice for the same shape in another layout.
    base_tn = gplan(BF16, T_, N_, 4096, 4096, 4096)[1]["kernel_id"]
    nt = _kid("bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4")
    assert gplan(BF16, N_, T_, 4096, 4096, 4096)[1]["kernel_id"] == nt
    assert gplan(BF16, T_, N_, 4096, 4096, 4096)[1]["kernel_id"] == base_tn != nt
    # The fp8 entry overrides the ring for A stored K x M, and for no other layout.
    gen = _kid("fp8_general_128x128x16")
    assert gplan(FP8, T_, N_, 2048, 2048, 2048)[1]["kernel_id"] == gen
    assert gplan(FP8, N_, N_, 2048, 2048, 2048)[1]["kernel_id"] != gen
    out = tmp_path / "saved.txt"
    assert tg.gemm_tuning_save(str(out)) == OK
    tg.gemm_tuning_clear()
    assert tg.gemm_tuning_load(str(out)) == 2
    assert gplan(FP8, T_, N_, 2048, 2048, 2048)[1]["kernel_id"] == gen
    tg.gemm_tuning_clear()
    bad = tmp_path / "bad_op.txt"
    bad.write_text("# libgemm tuning table v2\n2 2 0 64 64 64 16 16 0 fp8_general_128x128x16 0 0.3\n")
    assert tg.gemm_tuning_load(str(bad)) == -1 and tg.gemm_tuning_count() == 0
    # A v1 line under a v2 header has too few fields.
    bad.write_text("# libgemm tuning table v2\n0 1024 1024 1024 4 4 0 f32_mfma32_128x128x16_w2x2_a4b4 0 0.5\n")
    assert tg.gemm_tuning_load(str(bad)) == -1


def test_tuning_table_entry_that_cannot_run_is_ignored(tmp_path):
    """A recorded kernel that cannot run the call (here a split-K kernel
    recorded under the no-workspace key) is ignored: the built-in rules choose."""
    tg.gemm_tuning_clear()
    f = tmp_path / "t.txt"
    f.write_text("0 16 8192 8192 4 4 0 f32_skinny_splitk_n128_a4_w8_u1 0 0.04\n")
    assert tg.gemm_tuning_load(str(f)) == 1
    st, p = plan(F32, 16, 8192, 8192)
    assert st == OK and p["path"] == tg.GEMM_PATH_SKINNY
    tg.gemm_tuning_clear()


def test_tuning_load_errors(tmp_path):
    tg.gemm_tuning_clear()
    assert tg.gemm_tuning_load(str(tmp_path / "missing.txt")) == -1
    bad = tmp_path / "bad.txt"
    bad.write_text("0 16 16\n")
    assert tg.gemm_tuning_load(str(bad)) == -1
    assert tg.gemm_tuning_count() == 0
    assert tg.gemm_tuning_save(str(tmp_path / "no_dir" / "x.txt")) == tg.GEMM_ERR_INVALID_ARG
    # Autotune validates its arguments before touching a device.
    st, _ = tg.gemm_autotune(F32, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, 0, 0)
    assert st == tg.GEMM_ERR_INVALID_ARG                 # reps must be 1..1000
    st, _ = tg.gemm_autotune(F32, -1, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, 0, 5)
    assert st == tg.GEMM_ERR_INVALID_ARG
    st, p = tg.gemm_autotune(F32, 0, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, 0, 5)
    assert st == OK and p["path"] == tg.GEMM_PATH_NONE   # nothing to tune, no device needed
    st, _ = tg.gemm_autotune_general(FP8, N_, T_, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, 0, 0)
    assert st == tg.GEMM_ERR_INVALID_ARG
    st, _ = tg.gemm_autotune_general(FP8, N_, 2, 64, 64, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 64, 0, 0, 5)
    assert st == tg.GEMM_ERR_INVALID_ARG
    st, _ = tg.gemm_autotune_general(FP8, T_, N_, 64, 64, 64, 1.0, PA, 32, PB, 64, 0.0, PC, 64, 0, 0, 5)
    assert st == tg.GEMM_ERR_INVALID_ARG                 # A stored K x M needs lda >= M
    st, p = tg.gemm_autotune_general(BF16, T_, T_, 64, 0, 64, 1.0, PA, 64, PB, 64, 0.0, PC, 1, 0, 0, 5)
    assert st == OK and p["path"] == tg.GEMM_PATH_NONE


# ----------------------------------------------------------------------------- operand layouts and fp8

def gplan(dtype, op_a, op_b, M, N, K, alpha=1.0, A=PA, lda=None, B=PB, ldb=None, beta=0.0, C=PC, ldc=None,
          force=0, ws=0):
    lda = max(K if op_a == N_ else M, 1) if lda is None else lda
    ldb = max(N if op_b == N_ else K, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return tg.gemm_plan_query_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force, ws)


def kname(pl):
    return tg.gemm_kernel_query(pl["kernel_id"])["name"]


def test_every_dtype_and_layout_has_a_kernel():
    ks = tg.kernels()
    for dt in (F32, BF16, FP8):
        for bit in range(4):
            assert any(k["dtype"] == dt and (k["layouts"] >> bit) & 1 for k in ks), (dt, bit)


@pytest.mark.parametrize("dtype", [F32, BF16, FP8])
def test_general_validation(dtype):
    assert gplan(dtype, 2, N_, 4, 4, 4)[0] == INVALID
    assert gplan(dtype, N_, -1, 4, 4, 4)[0] == INVALID
    # op_a = T: A is K x M, lda >= M; op_b = T: B is N x K, ldb >= K.
    assert gplan(dtype, T_, N_, 8, 4, 4, lda=4)[0] == INVALID
    assert gplan(dtype, T_, N_, 8, 4, 4, lda=8)[0] == OK
    assert gplan(dtype, N_, T_, 4, 8, 6, ldb=5)[0] == INVALID
    assert gplan(dtype, N_, T_, 4, 8, 6, ldb=6)[0] == OK
    assert gplan(7, N_, N_, 4, 4, 4)[0] == INVALID


def test_general_nn_matches_plain_query():
    for dt in (F32, BF16):
        for (M, N, K) in [(4096, 4096, 4096), (1000, 3000, 777), (16, 8192, 8192), (300, 260, 264)]:
            a = plan(dt, M, N, K)
            b = gplan(dt, N_, N_, M, N, K)
            assert a == b, (dt, M, N, K)


def test_nt_takes_the_ring_kernels():
    st, pl = gplan(FP8, N_, T_, 8192, 8192, 8192)
    assert st == OK and kname(pl) == "fp8_mfma32_256x256x128_w2x2_nt_lines", pl
    assert pl["grid"] == 32 * 32 and pl["splits"] == 1
    st, pl = gplan(FP8, N_, T_, 8192, 8192, 512)      # below the whole-line kernel's K minimum
    assert st == OK and kname(pl) == "fp8_mfma32_256x256x64_w2x2_nt_ring4", pl
    # bf16 with B stored N x K: the whole-line kernel from K = 1024, the ring below.
    st, pl = gplan(BF16, N_, T_, 8192, 8192, 8192)
    assert st == OK and kname(pl) == "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines", pl
    # Both need only 16-byte rows of B^T: N is free.  Fewer 256^2 tiles than
    # compute units: the 128^2 whole-line kernel (from K = 256).
    st, pl = gplan(BF16, N_, T_, 4000, 4001, 1040)
    assert st == OK and kname(pl) == "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines", pl
    st, pl = gplan(BF16, N_, T_, 4000, 4001, 1000)
    assert st == OK and kname(pl) == "bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4", pl
    for K in (1040, 1000):
        st, pl = gplan(BF16, N_, T_, 1000, 1001, K)
        assert st == OK and kname(pl) == "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines", pl
    st, pl = gplan(BF16, N_, T_, 1000, 1001, 1044)
    assert st == OK and kname(pl) == "bf16_general_128x128x16", pl


@pytest.mark.parametrize("why", ["K", "lda", "ldb", "A", "B"])
def test_fp8_nt_unaligned_falls_back_to_general(why):
    kw = dict(M=512, N=512, K=1024)
    if why == "K":
        kw["K"] = 1000
    elif why == "lda":
        kw["lda"] = 1032 - 4
    elif why == "ldb":
        kw["ldb"] = 1024 + 8
    elif why == "A":
        kw["A"] = PA + 8
    else:
        kw["B"] = PB + 4
    st, pl = gplan(FP8, N_, T_, **kw)
    assert st == OK and kname(pl) == "fp8_general_128x128x16", (why, pl)


@pytest.mark.parametrize("dtype,prefix", [(F32, "f32"), (BF16, "bf16"), (FP8, "fp8")])
@pytest.mark.parametrize("ops", [(N_, T_), (T_, N_), (T_, T_), (N_, N_)])
def test_layouts_without_a_fast_kernel_take_general(dtype, prefix, ops):
    st, pl = gplan(dtype, ops[0], ops[1], 1000, 3000, 784)      # K a multiple of 16: fast kernels can run
    assert st == OK
    fast = dtype in (F32, BF16) or (dtype == FP8 and ops == (N_, T_))
    if fast:
        assert "general" not in kname(pl), pl
    else:
        assert kname(pl) == f"{prefix}_general_128x128x16", pl


def test_forcing_a_kernel_checks_its_layout():
    ring = [k["id"] for k in tg.kernels() if k["name"] == "fp8_mfma32_256x256x64_w2x2_nt_ring4"][0]
    assert gplan(FP8, N_, N_, 512, 512, 512, force=ring)[0] == UNSUP
    assert gplan(FP8, N_, T_, 512, 512, 512, force=ring)[0] == OK
    f32_ring = [k["id"] for k in tg.kernels() if k["name"] == "f32_mfma32_256x256x16_w2x2_a4b4_ring4"][0]
    assert gplan(F32, T_, N_, 512, 512, 512, force=f32_ring)[0] == UNSUP


@pytest.mark.parametrize("dtype", [F32, BF16, FP8])
@pytest.mark.parametrize("ops", [(N_, T_), (T_, N_), (T_, T_)])
def test_transposed_layouts_split_k(dtype, ops):
    M, N, K = 256, 512, 6000
    ws = tg.gemm_workspace_size(dtype, M, N, K)
    assert ws > 0
    st, pl = gplan(dtype, ops[0], ops[1], M, N, K, ws=ws)
    assert st == OK and pl["splits"] > 1, pl


def test_fp8_workspace_size():
    assert tg.gemm_workspace_size(FP8, 256, 512, 6000) == tg.gemm_workspace_size(BF16, 256, 512, 6000) > 0
    assert tg.gemm_workspace_size(FP8, 16, 8192, 8192) > 0


# ----------------------------------------------------------------------------- last-wave split

F32_RING256 = "f32_mfma32_256x256x16_w2x2_a4b4_ring4"


def test_wave_tail_plan():
    """272 tiles of 256 = one full wave + 16: the top 4096 rows run as one
    wave and the last tile row runs K-split (bf16 by choice, fp32 on the
    forced 256 x 256 ring, whose own choice is 128 x 128 tiles)."""
    for dtype, force in [(BF16, 0), (F32, kernel_ids(name=F32_RING256)[0])]:
        ws = tg.gemm_workspace_size(dtype, 4352, 4096, 4096)
        st, pl = plan(dtype, 4352, 4096, 4096, ws=ws, force=force)
        assert st == OK and pl["tile_m"] == 256 and pl["split_row"] == 4096 and pl["splits"] >= 2, pl
        assert pl["grid"] == 256 + 16 * pl["splits"]
        assert ws >= pl["splits"] * 256 * 4096 * 4
        # No workspace, or one too small: the plain plan.
        assert plan(dtype, 4352, 4096, 4096, force=force)[1]["split_row"] == 0
        assert plan(dtype, 4352, 4096, 4096, ws=1024, force=force)[1]["split_row"] == 0


def test_wave_tail_only_for_a_mostly_empty_last_wave():
    ws = 1 << 32
    ring = kernel_ids(name=F32_RING256)[0]
    assert plan(F32, 4096, 4096, 4096, ws=ws)[1]["split_row"] == 0           # exactly one wave
    assert plan(F32, 4096 + 256 * 13, 4096, 4096, ws=ws)[1]["split_row"] == 0  # 464 tiles: last wave 81% full
    assert plan(F32, 4352, 4096, 1024, ws=ws, force=ring)[1]["split_row"] == 0  # K too shallow to split
    st, pl = plan(BF16, 8448, 8192, 8192, ws=ws)
    assert st == OK and pl["split_row"] == 8192 and pl["splits"] >= 2, pl
    # 128 x 128 tiles run two to a compute unit: no last-wave split for them.
    for name in ["f32_mfma32_128x128x16_w2x2_a4b4_ring4", "bf16_mfma32_128x128x64_w2x2_a8b8_lines"]:
        st, pl = plan(F32 if name[0] == "f" else BF16, 4352, 4096, 4096, ws=ws, force=kernel_ids(name=name)[0])
        assert st == OK and pl["split_row"] == 0 and pl["splits"] == 1, pl


@pytest.mark.parametrize("dtype,ops,force", [(F32, (T_, N_), "f32_mfma32_256x256x16_w2x2_a4b4_tn_ring4"),
                                             (BF16, (N_, T_), ""),
                                             (FP8, (N_, T_), "fp8_mfma32_256x256x128_w2x2_nt_lines")])
def test_wave_tail_other_layouts(dtype, ops, force):
    M, N = 4352, 4096                           # 17 x 16 tiles of 256: one wave + 16
    ws = tg.gemm_workspace_size(dtype, M, N, 4096)
    st, pl = gplan(dtype, ops[0], ops[1], M, N, 4096, ws=ws, force=kernel_ids(name=force)[0] if force else 0)
    assert st == OK and pl["split_row"] > 0 and pl["splits"] >= 2, pl


@pytest.mark.parametrize("dtype,ops,shape,ws,expect", [
    # fp32: 128^2 tiles once a quarter of the last 256^2 wave is empty, with or without a workspace.
    (F32, (N_, N_), (4352, 4096, 4096), False, "f32_mfma32_128x128x16_w2x2_a4b4_ring4"),
    (F32, (N_, N_), (4352, 4096, 4096), True, "f32_mfma32_128x128x16_w2x2_a4b4_ring4"),
    (F32, (N_, N_), (2048, 11008, 4096), False, "f32_mfma32_128x128x16_w2x2_a4b4_ring4"),
    (F32, (N_, T_), (3072, 6144, 4096), True, "f32_mfma32_128x128x16_w2x2_a4b4_nt_ring4"),
    (F32, (N_, N_), (4096, 7168, 4096), False, "f32_mfma32_128x128x16_w2x2_a4b4_ring4"),     # 448 tiles
    (F32, (N_, N_), (4096 + 256 * 13, 4096, 4096), False, F32_RING256),                     # 464: 81% full
    (F32, (N_, N_), (4096, 4096, 4096), True, F32_RING256),                                 # whole wave
    # bf16 and the fp8 whole-line kernel: only between one and two waves, the second at most a quarter used.
    (BF16, (N_, N_), (3072, 6144, 4096), False, "bf16_mfma32_128x128x64_w2x2_a8b8_lines"),
    (BF16, (T_, N_), (4096, 5120, 4096), False, "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines"),
    (BF16, (N_, N_), (2048, 11008, 4096), False, "bf16_mfma32_256x256x64_w2x2_a8b8_lines"),  # 344 tiles
    (BF16, (N_, T_), (6144, 6144, 4096), False, "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines"),  # 576 tiles
    (BF16, (N_, N_), (3072, 6144, 4096), True, "bf16_mfma32_256x256x64_w2x2_a8b8_lines"),   # the split stays
    (BF16, (N_, N_), (8192, 8192, 8192), False, "bf16_mfma32_256x256x64_w2x2_a8b8_lines"),
    (FP8, (N_, T_), (4096, 5120, 4096), True, "fp8_mfma32_128x128x128_w2x2_nt_lines"),
    (FP8, (N_, T_), (2048, 11008, 4096), False, "fp8_mfma32_256x256x128_w2x2_nt_lines"),
    # the fp8 rings: as fp32, and on whole waves with K <= 2048.
    (FP8, (N_, N_), (6144, 6144, 4096), True, "fp8_mfma32_128x128x64_w2x2_nn_ring4"),
    (FP8, (T_, T_), (2048, 11008, 4096), False, "fp8_mfma32_128x128x64_w2x2_tt_ring4"),
    (FP8, (T_, N_), (4096, 4096, 1024), False, "fp8_mfma32_128x128x64_w2x2_tn_ring4"),
    (FP8, (N_, N_), (4096, 4096, 4096), False, "fp8_mfma32_256x256x64_w2x2_nn_ring4"),
])
def test_last_wave_takes_128_tiles(dtype, ops, shape, ws, expect):
    M, N, K = shape
    wsb = tg.gemm_workspace_size(dtype, M, N, K) if ws else 0
    st, pl = gplan(dtype, ops[0], ops[1], M, N, K, ws=wsb)
    assert st == OK and kname(pl) == expect, (kname(pl), pl)
    if expect != "bf16_mfma32_256x256x64_w2x2_a8b8_lines" or not ws:
        assert pl["split_row"] == 0


@pytest.mark.parametrize("ops,name", [((N_, T_), "nt"), ((T_, N_), "tn"), ((T_, T_), "tt")])
def test_bf16_transposed_layouts_take_their_rings(ops, name):
    st, pl = gplan(BF16, ops[0], ops[1], 8192, 8192, 8192)
    expect = {"nt": "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines", "tn": "bf16_mfma32_256x256x32_w2x2_a8b8_tn_lines",
              "tt": "bf16_mfma32_256x256x32_w2x2_a8b8_tt_ring4"}[name]
    assert st == OK and kname(pl) == expect, pl
    st, pl = gplan(BF16, ops[0], ops[1], 8192, 8192, 512)      # below the whole-line kernel's K minimum
    assert st == OK and kname(pl) == f"bf16_mfma32_256x256x32_w2x2_a8b8_{name}_ring4", pl
    # A^T rows are M long: M not a multiple of 8 leaves only the general kernel.
    if ops[0] == T_:
        st, pl = gplan(BF16, ops[0], ops[1], 8196, 8192, 8192)
        assert st == OK and kname(pl) == "bf16_general_128x128x16", pl


# ----------------------------------------------------------------------------- bf16 skinny

def test_bf16_skinny_with_workspace():
    for M in (1, 7, 16):
        ws = tg.gemm_workspace_size(BF16, M, 8192, 8192)
        assert ws >= 4 * M * 8192 * 4               # at least 4 splits of M x N fp32 partials
        st, pl = plan(BF16, M, 8192, 8192, ws=ws)
        assert st == OK and pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK and pl["grid"] == 64 * 4, pl
        assert kname(pl) == "bf16_skinny_lds_n128_w4_s4"
    # A not 16-byte aligned: the tiled kernels.
    st, pl = plan(BF16, 16, 8192, 8192, A=PA + 2, ws=1 << 30)
    assert st == OK and pl["path"] == tg.GEMM_PATH_TILED, pl
    # Without a workspace a split is impossible: the same kernel over the whole of K
    # (one workgroup per 128-column strip), unless no split is needed anyway.
    st, pl = plan(BF16, 16, 8192, 8192)
    assert st == OK and kname(pl) == "bf16_skinny_lds_n128_w4_s4_whole_k" and pl["grid"] == 64, pl
    assert pl["path"] == tg.GEMM_PATH_SKINNY
    assert plan(BF16, 16, 32768, 8192)[1]["path"] == tg.GEMM_PATH_SKINNY_SPLITK
    # B rows must be whole 16-byte chunks; M = 17 is not skinny.
    assert plan(BF16, 16, 8196, 8192, ws=1 << 30)[1]["path"] == tg.GEMM_PATH_TILED
    assert plan(BF16, 17, 8192, 8192, ws=1 << 30)[1]["path"] == tg.GEMM_PATH_TILED


# ----------------------------------------------------------------------------- skinny, B stored N x K

@pytest.mark.parametrize("dtype,prefix,chunk", [(F32, "f32", 4), (BF16, "bf16", 8), (FP8, "fp8", 16)])
def test_skinny_nt_choice(dtype, prefix, chunk):
    # 256 strips of 32 columns cover the chip: no split, no workspace needed.
    for M in (1, 9, 16):
        st, pl = gplan(dtype, N_, T_, M, 8192, 8192)
        assert st == OK and kname(pl) == f"{prefix}_skinny_nt_n32_w8_u2", pl
        assert pl["path"] == tg.GEMM_PATH_SKINNY and pl["grid"] == 256
    # With a workspace and few strips: K split across workgroups.
    ws = tg.gemm_workspace_size(dtype, 16, 1024, 8192)
    assert ws >= 8 * 16 * 1024 * 4
    st, pl = gplan(dtype, N_, T_, 16, 1024, 8192, ws=ws)
    assert st == OK and kname(pl) == f"{prefix}_skinny_nt_splitk_n32_w8_u2" and pl["grid"] == 32 * 8, pl
    # The same shape with the workspace of a call that needs no split: plain.
    st, pl = gplan(dtype, N_, T_, 16, 8192, 8192, ws=tg.gemm_workspace_size(dtype, 16, 8192, 8192))
    assert st == OK and kname(pl) == f"{prefix}_skinny_nt_n32_w8_u2", pl
    # M = 17, rows that are not whole 16-byte chunks, or op_a = T: not the skinny kernel.
    for kw in (dict(M=17), dict(K=8192 + chunk // 2), dict(ldb=8192 + chunk // 2), dict(B=PB + 4 * (dtype == BF16) + 8)):
        args = dict(M=16, N=8192, K=8192)
        args.update(kw)
        st, pl = gplan(dtype, N_, T_, **args)
        assert st == OK and "skinny_nt" not in kname(pl), (kw, kname(pl))
    st, pl = gplan(dtype, T_, T_, 16, 8192, 8192)
    assert st == OK and "skinny_nt" not in kname(pl)


def test_skinny_a_transposed_choice():
    """fp32 with A stored K x M and M <= 16: the streaming kernels that read
    A transposed, split over K when a workspace is passed; never for other
    layouts, M = 17, or K rows of A beyond 2^31 bytes."""
    for M in (1, 16):
        st, pl = gplan(F32, T_, N_, M, 8192, 8192, lda=16)      # (lda = 1 at M = 1 runs untransposed)
        assert st == OK and kname(pl) == "f32_skinny_mfma16_n2_at_w8_u4" and pl["grid"] == 256, pl
    st, pl = gplan(F32, T_, N_, 16, 8192, 8192, ws=tg.gemm_workspace_size(F32, 16, 8192, 8192))
    assert st == OK and kname(pl) == "f32_skinny_splitk_n128_at_w8_u1" and pl["grid"] == 256, pl
    assert "_at_" not in kname(plan(F32, 16, 8192, 8192)[1])
    assert "_at_" not in kname(gplan(F32, T_, N_, 17, 8192, 8192)[1])
    assert "_at_" not in kname(gplan(F32, T_, T_, 16, 8192, 8192)[1])
    # bf16: the streaming kernel reading A's K rows in 16-byte chunks (M and
    # lda multiples of 8, A 16-byte aligned), over the whole of K or split.
    st, pl = gplan(BF16, T_, N_, 16, 8192, 8192, lda=16)
    assert st == OK and kname(pl) == "bf16_skinny_lds_n128_at_w4_s4_whole_k" and pl["grid"] == 64, pl
    st, pl = gplan(BF16, T_, N_, 8, 8192, 8192, lda=8, ws=tg.gemm_workspace_size(BF16, 8, 8192, 8192))
    assert st == OK and kname(pl) == "bf16_skinny_lds_n128_at_w4_s4" and pl["grid"] == 256, pl
    # Otherwise (rows of A not whole 16-byte chunks): the same kernel loading
    # A 2 bytes a lane.
    at1 = "bf16_skinny_lds_n128_at1_w4_s4"
    assert kname(gplan(BF16, T_, N_, 5, 8192, 8192, lda=8)[1]) == at1 + "_whole_k"   # rows of 5
    assert kname(gplan(BF16, T_, N_, 16, 8192, 8192, lda=20)[1]) == at1 + "_whole_k"
    assert kname(gplan(BF16, T_, N_, 16, 8192, 8192, lda=16, A=PA + 2)[1]) == at1 + "_whole_k"
    st, pl = gplan(BF16, T_, N_, 12, 8192, 8192, lda=13, ws=tg.gemm_workspace_size(BF16, 12, 8192, 8192))
    assert st == OK and kname(pl) == at1 and pl["grid"] == 256, pl
    assert "_at" not in kname(gplan(BF16, N_, N_, 16, 8192, 8192)[1])
    assert "_at" not in kname(gplan(BF16, T_, N_, 17, 8192, 8192, lda=17)[1])
    K = 1 << 20
    st, pl = gplan(F32, T_, N_, 16, 64, K, lda=1 << 9)             # ((K - 1) * lda + M) * 4 < 2^31
    assert st == OK and kname(pl) == "f32_skinny_mfma16_n2_at_w8_u4", pl
    st, pl = gplan(F32, T_, N_, 16, 64, K, lda=(1 << 9) + 4)       # > 2^31
    assert st == OK and "_at_" not in kname(pl), pl
    # Forced on untransposed A they refuse, as the untransposed ones do here.
    for n in ("f32_skinny_mfma16_n2_at_w8_u4", "f32_skinny_splitk_n128_at_w8_u1"):
        assert plan(F32, 16, 8192, 8192, force=_kid(n), ws=1 << 30)[0] == UNSUP
    assert gplan(F32, T_, N_, 16, 8192, 8192, force=_kid("f32_skinny_mfma16_n2_a4_w8_u4"))[0] == UNSUP


def test_skinny_nt_largest_leading_dimension():
    # A workgroup's 32 rows of B^T and the 16 rows of A must each span less
    # than 2^31 bytes for the kernel's 32-bit offsets; beyond that another
    # kernel takes the call.
    ld = (1 << 24) - 4096
    st, pl = gplan(F32, N_, T_, 16, 64, 8192, lda=ld, ldb=ld)
    assert st == OK and "skinny_nt" in kname(pl), pl
    st, pl = gplan(F32, N_, T_, 16, 64, 8192, ldb=(1 << 24) + (1 << 20))
    assert st == OK and "skinny_nt" not in kname(pl), pl


def test_skinny_nt_forced_needs_its_layout():
    for k in tg.kernels():
        if "skinny_nt" not in k["name"]:
            continue
        assert k["layouts"] == 2
        st, _ = plan(k["dtype"], 16, 8192, 8192, force=k["id"], ws=1 << 30)
        assert st == UNSUP, k["name"]
        st, _ = gplan(k["dtype"], N_, T_, 16, 8192, 8192, force=k["id"], ws=1 << 30)
        assert st == OK, k["name"]


# ----------------------------------------------------------------------------- output quantisation

def eplan(dtype, op_a, op_b, M, N, K, out_type, ws=0, force=0, C=PC, beta=0.0, ldo=None, out=0x7f3000000000):
    lda = K if op_a == N_ else M
    ldb = N if op_b == N_ else K
    epi = (0, 0, out_type, out, N if ldo is None else ldo, 0.0)
    return tg.gemm_plan_query_epi(dtype, op_a, op_b, M, N, K, 1.0, PA, lda, PB, ldb, beta, C, N, force, epi, ws)


def test_output_types_of_the_kernels():
    outs = {k["name"]: k["outputs"] for k in tg.kernels()}
    assert all(v & 1 for v in outs.values())
    for name in ("f32_mfma32_256x256x16_w2x2_a4b4_ring4", "bf16_mfma32_256x256x32_w2x2_a8b8_ring4",
                 "bf16_mfma32_256x256x64_w2x2_a8b8_lines", "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines",
                 "bf16_mfma32_256x256x32_w2x2_a8b8_tn_lines", "bf16_mfma32_128x128x64_w2x2_a8b8_lines",
                 "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines", "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines",
                 "bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4", "bf16_mfma32_256x256x32_w2x2_a8b8_tn_ring4",
                 "bf16_mfma32_256x256x32_w2x2_a8b8_tt_ring4", "fp8_mfma32_256x256x64_w2x2_nt_ring4",
                 "fp8_mfma32_256x256x128_w2x2_nt_lines", "fp8_mfma32_128x128x128_w2x2_nt_lines",
                 "fp8_mfma32_128x128x64_w2x2_nn_ring4", "fp8_mfma32_128x128x64_w2x2_tn_ring4",
                 "fp8_mfma32_128x128x64_w2x2_tt_ring4",
                 "f32_general_128x128x16", "bf16_general_128x128x16", "fp8_general_128x128x16",
                 "f32_skinny_splitk_n128_a4_w8_u1", "bf16_skinny_lds_n128_w4_s4", "bf16_skinny_lds_n128_w4_s4_whole_k", "bf16_skinny_nt_n32_w8_u2",
                 "fp8_skinny_nt_splitk_n32_w8_u2", "fp8_skinny_kn_n128_w4_s4", "fp8_skinny_kn_n128_w4_s4_whole_k",
                 "fp8_skinny_kn_at1_n128_w4_s3", "fp8_skinny_kn_at1_n128_w4_s3_whole_k",
                 "f32_skinny_tt_n32_w8_u2", "bf16_skinny_tt_splitk_n32_w8_u2", "fp8_skinny_tt_n32_w8_u2"):
        assert outs[name] == 7, name
    assert outs["f32_skinny_mfma16_n2_a4_w8_u4"] == 7 and outs["f32_mfma32_128x128x16_w2x2_a4b4"] == 7
    # Register-staged kernels holding 256 accumulators per lane write fp32 only.
    assert outs["f32_mfma32_256x256x16_w2x2_a4b4"] == 1 and outs["bf16_mfma32_256x256x64_w2x2_a8b8_pipe"] == 1


@pytest.mark.parametrize("out_type", [tg.GEMM_OUT_BF16, tg.GEMM_OUT_FP8])
def test_output_quantisation_choice(out_type):
    # The main shapes keep their kernels, and C may be NULL when beta == 0.
    for dt, M, N, K, name in ((F32, 4096, 4096, 4096, "f32_mfma32_256x256x16_w2x2_a4b4_ring4"),
                              (BF16, 8192, 8192, 8192, "bf16_mfma32_256x256x64_w2x2_a8b8_lines")):
        st, pl = eplan(dt, N_, N_, M, N, K, out_type, C=0)
        assert st == OK and kname(pl) == name, pl
    st, pl = eplan(FP8, N_, T_, 8192, 8192, 8192, out_type, C=0)
    assert st == OK and kname(pl) == "fp8_mfma32_256x256x128_w2x2_nt_lines"
    st, pl = eplan(BF16, N_, T_, 16, 8192, 8192, out_type, C=0)
    assert st == OK and kname(pl) == "bf16_skinny_nt_n32_w8_u2"
    # Short K: the 256-tile kernels preferred there write fp32 only, so a
    # regular kernel that writes the type runs, never the general fallback.
    st, pl = eplan(BF16, N_, N_, 4096, 4096, 512, out_type, C=0)
    info = tg.gemm_kernel_query(pl["kernel_id"])
    assert st == OK and "general" not in info["name"] and (info["outputs"] >> out_type) & 1, pl
    assert kname(gplan(BF16, N_, N_, 4096, 4096, 512)[1]) == "bf16_mfma32_256x256x64_w2x2_a8b8_pipe"
    # fp32 M <= 16 without a workspace: the one-pass skinny kernel.
    st, pl = eplan(F32, N_, N_, 16, 8192, 8192, out_type)
    assert st == OK and pl["path"] == tg.GEMM_PATH_SKINNY, pl
    st, pl = eplan(F32, N_, N_, 16, 8192, 8192, out_type, ws=tg.gemm_workspace_size(F32, 16, 8192, 8192))
    assert st == OK and kname(pl) == "f32_skinny_splitk_n128_a4_w8_u1"
    # A kernel that writes fp32 only cannot be forced.
    only_f32 = [k["id"] for k in tg.kernels() if k["outputs"] == 1 and k["dtype"] == F32 and k["layouts"] & 1]
    assert only_f32
    for kid in only_f32:
        assert eplan(F32, N_, N_, 16, 512, 512, out_type, force=kid)[0] == UNSUP
        assert eplan(F32, N_, N_, 16, 512, 512, tg.GEMM_OUT_F32, force=kid)[0] == OK


def test_output_quantisation_validation():
    assert eplan(F32, N_, N_, 64, 64, 64, 3)[0] == INVALID
    assert eplan(F32, N_, N_, 64, 64, 64, -1)[0] == INVALID
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_BF16, ldo=63)[0] == INVALID
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_BF16, out=0)[0] == INVALID
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_BF16, out=0x7f3000000001)[0] == INVALID   # bf16 needs 2-byte
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_FP8, out=0x7f3000000001)[0] == OK
    # C is needed as C0 when beta != 0, and always for fp32 output.
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_BF16, C=0, beta=0.5)[0] == INVALID
    assert eplan(F32, N_, N_, 64, 64, 64, tg.GEMM_OUT_F32, C=0)[0] == INVALID
    assert eplan(F32, N_, N_, 0, 64, 64, tg.GEMM_OUT_BF16, out=0)[0] == OK       # empty: nothing is written


@pytest.mark.parametrize("ops,name", [((N_, N_), "fp8_mfma32_256x256x64_w2x2_nn_ring4"),
                                      ((T_, N_), "fp8_mfma32_256x256x64_w2x2_tn_ring4"),
                                      ((T_, T_), "fp8_mfma32_256x256x64_w2x2_tt_ring4")])
def test_fp8_other_layouts_take_their_rings(ops, name):
    st, pl = gplan(FP8, ops[0], ops[1], 8192, 8192, 8192)
    assert st == OK and kname(pl) == name and pl["grid"] == 32 * 32, pl
    # Rows of the K x M / K x N operand must be whole 16-byte chunks.
    bad = dict(M=8192 + 8) if ops[0] == T_ else dict(N=8192 + 8)
    args = dict(M=8192, N=8192, K=8192)
    args.update(bad)
    st, pl = gplan(FP8, ops[0], ops[1], **args)
    assert st == OK and kname(pl) == "fp8_general_128x128x16", pl


# ----------------------------------------------------------------------------- no-allocation entry point

def _noalloc(dtype, M, N, K, lda=None, ldb=None, ldc=None, A=PA, B=PB, C=PC, op_a=0, op_b=0):
    lda = (max(K, 1) if op_a == 0 else max(M, 1)) if lda is None else lda
    ldb = (max(N, 1) if op_b == 0 else max(K, 1)) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return tg.gemm_general_noalloc(dtype, op_a, op_b, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, 0, None, 0)


def test_noalloc_checks_arguments_before_anything_else():
    # Invalid arguments are reported as by gemm_general, with no HIP call (no GPU here).
    assert _noalloc(F32, -1, 4, 4) == tg.GEMM_ERR_INVALID_ARG
    assert _noalloc(F32, 4, 4, 4, lda=3) == tg.GEMM_ERR_INVALID_ARG
    assert _noalloc(7, 4, 4, 4) == tg.GEMM_ERR_INVALID_ARG
    assert _noalloc(F32, 4, 4, 4, A=0) == tg.GEMM_ERR_INVALID_ARG
    # Empty problems are a no-op.
    assert _noalloc(F32, 0, 4, 4) == tg.GEMM_OK
    assert _noalloc(BF16, 4, 0, 4) == tg.GEMM_OK


def test_noalloc_rejects_problems_beyond_the_static_scratch():
    assert tg.GEMM_STATIC_SCRATCH_BYTES == 32 << 20
    # A 2048 x 2048 bf16 problem with a deep K splits 4 ways: 64 MiB of partial products.
    need = tg.gemm_workspace_size(BF16, 2048, 2048, 65536)
    assert need > tg.GEMM_STATIC_SCRATCH_BYTES
    assert _noalloc(BF16, 2048, 2048, 65536) == tg.GEMM_ERR_SCRATCH
    assert "static scratch" in tg.gemm_status_string(tg.GEMM_ERR_SCRATCH)
    # The decode and small-tile splits fit.
    for dt, M, N, K in [(F32, 16, 8192, 8192), (BF16, 16, 8192, 8192), (BF16, 512, 512, 8192), (F32, 16, 16384, 65536)]:
        assert 0 < tg.gemm_workspace_size(dt, M, N, K) <= tg.GEMM_STATIC_SCRATCH_BYTES, (dt, M, N, K)


def test_f32_ring64_is_the_choice_for_config_4a():
    """fp32 1000 x 3000 x 777 (rows of A 4-byte aligned only) takes the 64 x 64
    ring with 4-byte A loads, with or without a workspace."""
    for ws in (0, 1 << 30):
        st, pl = tg.gemm_plan_query(F32, 1000, 3000, 777, 2.0, 0x1000, 777, 0x1000, 3000, -1.0,
                                    0x1000, 3000, 0, ws)
        assert st == OK and kname(pl) == \
            "f32_mfma32_64x64x16_w2x2_a1b4_ring6", pl


# ----------------------------------------------------------------------------- fp8 skinny, B stored K x N

def test_fp8_kn_skinny_choice_and_workspace():
    """M <= 16 with fp8 weights stored K x N: without a workspace and with at
    most 128 strips of 128 columns, the streaming kernel over the whole of K;
    otherwise the 128^2 ring (split over K with a workspace).  The split form
    runs when forced and the workspace query covers it."""
    split = kernel_ids(name="fp8_skinny_kn_n128_w4_s4")[0]
    for M in (1, 7, 16):
        ws = tg.gemm_workspace_size(FP8, M, 8192, 8192)
        assert ws >= 4 * M * 8192 * 4               # 64 strips x 4 splits
        st, pl = gplan(FP8, N_, N_, M, 8192, 8192, ws=ws, force=split)
        assert st == OK and kname(pl) == "fp8_skinny_kn_n128_w4_s4" and pl["grid"] == 64 * 4, pl
        assert pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK
        st, pl = gplan(FP8, N_, N_, M, 8192, 8192)
        assert st == OK and kname(pl) == "fp8_skinny_kn_n128_w4_s4_whole_k" and pl["grid"] == 64, pl
        st, pl = gplan(FP8, N_, N_, M, 8192, 8192, ws=ws)
        assert st == OK and kname(pl) == "fp8_mfma32_128x128x64_w2x2_nn_ring4" and pl["splits"] > 1, pl
    assert kname(gplan(FP8, N_, N_, 16, 16384, 4096)[1]) == "fp8_skinny_kn_n128_w4_s4_whole_k"   # 128 strips
    assert kname(gplan(FP8, N_, N_, 16, 16512, 4096)[1]) == "fp8_mfma32_128x128x64_w2x2_nn_ring4"  # 129
    # Rows of B must be whole 16-byte chunks, M at most 16, A stored M x K.
    assert "skinny" not in kname(gplan(FP8, N_, N_, 16, 8200, 8192)[1])
    assert gplan(FP8, N_, N_, 17, 8192, 8192)[1]["path"] == tg.GEMM_PATH_TILED
    assert gplan(FP8, T_, N_, 16, 8192, 8192)[1]["path"] == tg.GEMM_PATH_TILED
    # K too short for two 512-deep slices: one split, which needs no workspace.
    st, pl = gplan(FP8, N_, N_, 16, 8192, 1008, force=split)
    assert st == OK and kname(pl) == "fp8_skinny_kn_n128_w4_s4" and pl["splits"] == 1, pl
    # A stored K x M: the byte-loading form where the 128^2 ring cannot run
    # (A's K rows not whole 16-byte chunks), split with a workspace.
    at1 = "fp8_skinny_kn_at1_n128_w4_s3"
    for M, lda in [(12, 12), (13, 13), (5, 16), (1, 3)]:
        assert kname(gplan(FP8, T_, N_, M, 8192, 8192, lda=lda)[1]) == at1 + "_whole_k"
        ws = tg.gemm_workspace_size(FP8, M, 8192, 8192)
        st, pl = gplan(FP8, T_, N_, M, 8192, 8192, lda=lda, ws=ws)
        assert st == OK and kname(pl) == at1 and pl["grid"] == 256, pl
    assert kname(gplan(FP8, T_, N_, 16, 8192, 8192, lda=16)[1]) == "fp8_mfma32_128x128x64_w2x2_tn_ring4"
    assert kname(gplan(FP8, T_, N_, 16, 8192, 8192, lda=16, A=PA + 1)[1]) == at1 + "_whole_k"
    assert kname(gplan(FP8, T_, T_, 12, 8192, 8192, lda=12)[1]) == "fp8_skinny_tt_n32_w8_u2"


@pytest.mark.parametrize("dtype", [F32, BF16, FP8])
def test_single_row_a_stored_transposed_runs_untransposed(dtype):
    """M = 1 with A stored K x 1 and lda = 1 is the same memory as a 1 x K
    row: it takes the untransposed layout's kernels (the streaming ones for
    B stored K x N and N x K); with lda > 1 it stays transposed."""
    for op_b in (N_, T_):
        st, pl = gplan(dtype, T_, op_b, 1, 8192, 8192, lda=1)
        st2, pl2 = gplan(dtype, N_, op_b, 1, 8192, 8192)
        assert st == st2 == OK and kname(pl) == kname(pl2) and pl["grid"] == pl2["grid"], (kname(pl), kname(pl2))
        if dtype != FP8 or op_b == T_:
            assert "skinny" in kname(pl), kname(pl)
        st, pl = gplan(dtype, T_, op_b, 1, 8192, 8192, lda=2)
        assert st == OK and ((tg.gemm_kernel_query(pl["kernel_id"])["layouts"] >> (2 + op_b)) & 1), kname(pl)
    # A forced kernel keeps the layout as passed.
    if dtype == F32:
        at = kernel_ids(name="f32_skinny_mfma16_n2_at_w8_u4")[0]
        st, pl = gplan(F32, T_, N_, 1, 8192, 8192, lda=1, force=at)
        assert st == OK and kname(pl) == "f32_skinny_mfma16_n2_at_w8_u4", pl


@pytest.mark.parametrize("dtype", [F32, BF16, FP8])
def test_skinny_tt_choice(dtype):
    """M <= 16 with A stored K x M and B stored N x K: the N x K streaming
    kernel gathering A, split over K with a workspace; fp8 with a workspace
    keeps the 128^2 ring split over K where A's rows allow it."""
    pre = {F32: "f32", BF16: "bf16", FP8: "fp8"}[dtype]
    for M, lda in [(16, 16), (12, 12), (5, 8), (1, 3)]:
        assert kname(gplan(dtype, T_, T_, M, 8192, 8192, lda=lda)[1]) == pre + "_skinny_tt_n32_w8_u2"
        ws = tg.gemm_workspace_size(dtype, M, 4096, 8192)        # 128 strips of 32 columns: split in two
        st, pl = gplan(dtype, T_, T_, M, 4096, 8192, lda=lda, ws=ws)
        ring = dtype == FP8 and (lda * M) % 16 == 0 and M % 16 == 0
        want = "fp8_mfma32_128x128x64_w2x2_tt_ring4" if ring else pre + "_skinny_tt_splitk_n32_w8_u2"
        assert st == OK and kname(pl) == want, (M, lda, kname(pl))
    assert "skinny" not in kname(gplan(dtype, T_, T_, 17, 8192, 8192, lda=17)[1])
