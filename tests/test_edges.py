"""GPU edge cases, checked against the oracle.

Exact-integer mode: operands are small integers (exact in fp32 and bf16) and
every partial sum is an integer below 2^24, so any summation order gives the
exact answer and the GPU must equal the oracle bit for bit.  That catches
indexing, edge and masking mistakes with zero tolerance.  Shapes straddle
the tile sizes (16, 32, 64, 128, 256) on every side, and every kernel in the
table is forced through them.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, needs_workspace, ratio, run_gemm, say

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def _shapes(seed, count):
    rng = np.random.default_rng(seed)
    allc = list(itertools.product(EDGE, EDGE, EDGE))
    pick = rng.choice(len(allc), size=count, replace=False)
    fixed = [(1, 1, 1), (257, 257, 257), (16, 257, 255), (129, 1, 65), (1, 300, 513), (300, 1, 2)]
    return fixed + [allc[i] for i in pick]


def _exact(A, B, C0, alpha, beta):
    return oracle.gemm_ref(host_view(A), host_view(B), alpha, beta, C0.numpy())


def _kernel_ids(dtype, path=None):
    """Kernels of this operand type that run untransposed operands (the layout these tests use)."""
    return [k["id"] for k in tg.kernels()
            if k["dtype"] == dtype and (path is None or k["path"] == path) and k["layouts"] & 1]


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_exact_integer_auto_choice(gpu_available, dtype):
    for i, (M, N, K) in enumerate(_shapes(7 if dtype == "f32" else 8, 60)):
        A, B, C0 = make_integer_inputs(M, N, K, seed=i, dtype=dtype)
        for alpha, beta in [(2.0, -1.0), (1.0, 0.0)]:
            say(f"[exact] {dtype} auto M={M} N={N} K={K} alpha={alpha} beta={beta} seed={i}")
            C, _, _ = run_gemm(A, B, C0, alpha, beta)
            np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, alpha, beta),
                                          err_msg=f"{dtype} {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_exact_integer_every_kernel(gpu_available, dtype):
    did = tg.GEMM_DTYPE_F32 if dtype == "f32" else tg.GEMM_DTYPE_BF16F32
    shapes = _shapes(11 if dtype == "f32" else 12, 14)
    for kid in _kernel_ids(did):
        info = tg.gemm_kernel_query(kid)
        for i, (M, N, K) in enumerate(shapes):
            if info["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK):
                M = min(M, 16)
            A, B, C0 = make_integer_inputs(M, N, K, seed=100 + i, dtype=dtype)
            wsb = tg.gemm_workspace_size(did, M, N, K) if needs_workspace(kid) else 0
            st, _ = tg.gemm_plan_query(did, M, N, K, 2.0, 0x1000, K, 0x1000, N, 0.5, 0x1000, N, kid, wsb)
            if st != tg.GEMM_OK:
                continue    # this kernel's vector width does not fit the shape
            say(f"[exact] kernel={info['name']} M={M} N={N} K={K} seed={100 + i}")
            C, _, _ = run_gemm(A, B, C0, 2.0, 0.5, kernel=kid)
            np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, 2.0, 0.5),
                                          err_msg=f"{info['name']} {M}x{N}x{K}")


def test_f32_ring_ragged_multi_wave(gpu_available):
    """The fp32 ring kernel on a problem with more tiles than compute units:
    4100 x 4300 gives 17 x 17 = 289 tiles of 256 x 256 (two waves, ragged
    last tiles) and K = 1100 gives 69 k slices of 16 (the last one
    partial; the ring runs on to a multiple of its depth with zero slices).
    Integer data: the result must equal the oracle exactly, with beta on and
    off, and with a C whose rows are not 16-byte aligned (scalar stores)."""
    M, N, K = 4100, 4300, 1100
    A, B, C0 = make_integer_inputs(M, N, K, seed=301)
    ring = [k for k in _kernel_ids(tg.GEMM_DTYPE_F32) if "ring" in tg.gemm_kernel_query(k)["name"]]
    assert ring
    for kid in ring:
        name = tg.gemm_kernel_query(kid)["name"]
        for alpha, beta, pad in [(2.0, 0.5, 0), (1.0, 0.0, 0), (-1.0, 1.0, 1)]:
            say(f"[ring multi-tile] kernel={name} M={M} N={N} K={K} alpha={alpha} beta={beta} c_pad={pad} seed=301")
            C, _, _ = run_gemm(A, B, C0, alpha, beta, kernel=kid, pad=(0, 0, pad))
            np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, alpha, beta),
                                          err_msg=f"{name} alpha={alpha} beta={beta} c_pad={pad}")


def test_bf16_ring_ragged_multi_wave(gpu_available):
    """The ring kernels (and the line-granular one) on a problem with more
    tiles than compute units:
    4100 x 4296 gives 17 x 17 = 289 tiles of 256 x 256 (two waves, ragged
    last tiles) and K = 1096 gives 35 k slices, the last one partial.
    Integer data: every ring kernel must equal the oracle exactly, with beta
    on and off."""
    M, N, K = 4100, 4296, 1096
    A, B, C0 = make_integer_inputs(M, N, K, seed=300, dtype="bf16f32")
    refs = {(2.0, 0.5): _exact(A, B, C0, 2.0, 0.5), (1.0, 0.0): _exact(A, B, C0, 1.0, 0.0)}
    ring = [k for k in _kernel_ids(tg.GEMM_DTYPE_BF16F32)
            if "ring" in tg.gemm_kernel_query(k)["name"] or "lines" in tg.gemm_kernel_query(k)["name"]]
    assert ring
    for kid in ring:
        name = tg.gemm_kernel_query(kid)["name"]
        for (alpha, beta), ref in refs.items():
            say(f"[ring multi-tile] kernel={name} M={M} N={N} K={K} alpha={alpha} beta={beta} seed=300")
            C, _, _ = run_gemm(A, B, C0, alpha, beta, kernel=kid)
            np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=f"{name} alpha={alpha} beta={beta}")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_random_values_every_kernel(gpu_available, dtype):
    """Full-precision random operands through every kernel on ragged shapes."""
    did = tg.GEMM_DTYPE_F32 if dtype == "f32" else tg.GEMM_DTYPE_BF16F32
    for kid in _kernel_ids(did):
        info = tg.gemm_kernel_query(kid)
        M = 16 if info["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK) else 300
        for (N, K) in [(520, 1030), (264, 96)]:
            A, B, C0 = make_random_inputs(M, N, K, seed=kid, dist="normal", dtype=dtype)
            wsb = tg.gemm_workspace_size(did, M, N, K) if needs_workspace(kid) else 0
            st, _ = tg.gemm_plan_query(did, M, N, K, 1.0, 0x1000, K, 0x1000, N, -2.0, 0x1000, N, kid, wsb)
            if st != tg.GEMM_OK:
                continue
            say(f"[random] kernel={info['name']} M={M} N={N} K={K} seed={kid}")
            C, _, _ = run_gemm(A, B, C0, 1.0, -2.0, kernel=kid)
            r = ratio(C, A, B, C0, 1.0, -2.0)
            assert r <= TOL[dtype], (info["name"], r)


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("M", [5, 16, 200])
def test_beta_zero_never_reads_C(gpu_available, dtype, M):
    """beta = 0 with C full of NaN: the result is finite and exact."""
    A, B, C0 = make_integer_inputs(M, 130, 70, seed=3, dtype=dtype)
    say(f"[nan-C] {dtype} M={M} N=130 K=70 beta=0")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.0, c_fill=float("nan"))
    assert np.isfinite(C).all()
    np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, 1.0, 0.0))


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("M,N,K", [(16, 200, 300), (130, 70, 90), (300, 260, 264)])
def test_padded_leading_dimensions_with_nan_padding(gpu_available, dtype, M, N, K):
    """lda/ldb/ldc wider than the matrix; NaN in the padding must not reach C,
    and C's padding (a guard band) must come back untouched."""
    A, B, C0 = make_integer_inputs(M, N, K, seed=4, dtype=dtype)
    for pad in [(3, 5, 7), (8, 8, 8), (1, 0, 2)]:
        say(f"[padded] {dtype} M={M} N={N} K={K} pad={pad}")
        C, Cd, cbuf = run_gemm(A, B, C0, 2.0, -1.0, pad=pad)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, 2.0, -1.0))
        ldc = N + pad[2]
        full = cbuf[:M * ldc].view(M, ldc)
        if pad[2]:
            assert torch.isnan(full[:, N:]).all(), "guard band of C was written"
        assert torch.isnan(cbuf[M * ldc:]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_unaligned_bases_take_element_loads(gpu_available, dtype):
    A, B, C0 = make_integer_inputs(140, 136, 136, seed=5, dtype=dtype)
    for off in [(1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 3, 2)]:
        say(f"[unaligned] {dtype} 140x136x136 offsets={off}")
        C, _, _ = run_gemm(A, B, C0, 1.0, 1.0, offset=off)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, 1.0, 1.0))


def test_skinny_rows_1_to_16(gpu_available):
    for M in range(1, 17):
        A, B, C0 = make_integer_inputs(M, 1000, 999, seed=M)
        say(f"[skinny] M={M} N=1000 K=999")
        C, _, _ = run_gemm(A, B, C0, -1.0, 2.0)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, -1.0, 2.0))


def test_skinny_lds_a_kernel_matches_direct_loads(gpu_available):
    """The single-pass kernel that stages A through LDS pairs the same k in
    the same order as the kernel that loads A straight into registers: on
    random data the two give the same bits, for row counts below 16, K not a
    multiple of its 512-deep batches (nor of 16) and ragged N; on integer
    data both equal the oracle."""
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    lds, direct = ids["f32_skinny_mfma16_n2_alds_w8_u4"], ids["f32_skinny_mfma16_n2_a4_w8_u4"]
    for M, N, K in [(16, 8192, 8192), (1, 1000, 1028), (7, 96, 516), (16, 32, 4), (13, 2050, 3000)]:
        A, B, C0 = make_random_inputs(M, N, K, seed=M + N + K, dist="uniform")
        st, pl = tg.gemm_plan_query(tg.GEMM_DTYPE_F32, M, N, K, 1.5, 0x1000, K, 0x1000, N, -0.5, 0x1000, N, 0, 0)
        assert st == tg.GEMM_OK and pl["kernel_id"] == lds, tg.gemm_kernel_query(pl["kernel_id"])["name"]
        say(f"[skinny lds A] M={M} N={N} K={K}")
        C1, _, _ = run_gemm(A, B, C0, 1.5, -0.5, kernel=lds)
        C2, _, _ = run_gemm(A, B, C0, 1.5, -0.5, kernel=direct)
        np.testing.assert_array_equal(C1, C2, err_msg=f"{M}x{N}x{K}")
        assert ratio(C1, A, B, C0, 1.5, -0.5) <= TOL["f32"]
        Ai, Bi, Ci = make_integer_inputs(M, N, K, seed=M * 7 + K)
        C, _, _ = run_gemm(Ai, Bi, Ci, -1.0, 2.0, kernel=lds)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(Ai, Bi, Ci, -1.0, 2.0), err_msg=f"{M}x{N}x{K}")
        # A and B inside wider NaN-padded rows (A's padding a multiple of 4, so
        # its rows stay 16-byte aligned), C padded by an odd amount.
        C, _, _ = run_gemm(Ai, Bi, Ci, -1.0, 2.0, kernel=lds, pad=(12, 6, 3))
        np.testing.assert_array_equal(C.astype(np.float64), _exact(Ai, Bi, Ci, -1.0, 2.0), err_msg=f"padded {M}x{N}x{K}")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_quick_returns(gpu_available, dtype):
    torch_dt = torch.float32 if dtype == "f32" else torch.bfloat16
    C0 = torch.arange(12, dtype=torch.float32).reshape(3, 4).cuda()
    A = torch.empty(3, 0, dtype=torch_dt, device="cuda")
    B = torch.empty(0, 4, dtype=torch_dt, device="cuda")
    say(f"[quick] {dtype} K=0")
    C = tg.gemm(A, B, C0.clone(), alpha=2.0, beta=0.5)
    torch.cuda.synchronize()
    assert torch.equal(C, 0.5 * C0)
    C = tg.gemm(A, B, torch.full((3, 4), float("nan"), device="cuda"), alpha=2.0, beta=0.0)
    torch.cuda.synchronize()
    assert torch.equal(C, torch.zeros(3, 4, device="cuda"))
    A = torch.full((3, 5), float("nan"), device="cuda").to(torch_dt)
    B = torch.full((5, 4), float("nan"), device="cuda").to(torch_dt)
    say(f"[quick] {dtype} alpha=0 with NaN operands")
    C = tg.gemm(A, B, C0.clone(), alpha=0.0, beta=-1.0)
    torch.cuda.synchronize()
    assert torch.equal(C, -C0)
    Cm = torch.full((0, 4), 1.0, device="cuda")
    tg.gemm(torch.empty(0, 5, dtype=torch_dt, device="cuda"), B, Cm)


def test_errors_surface_as_exceptions(gpu_available):
    A = torch.ones(4, 4, device="cuda")
    with pytest.raises(ValueError):
        tg.gemm(A, A.t(), torch.empty(4, 4, device="cuda"))   # column-major B rejected
    with pytest.raises(ValueError):
        tg.gemm(A, A, beta=1.0)
    st = tg.gemm_f32(4, 4, 4, 1.0, A.data_ptr(), 3, A.data_ptr(), 4, 0.0, A.data_ptr(), 4, 0)
    assert st == tg.GEMM_ERR_INVALID_ARG


def test_nonzero_mean_large_k_within_worst_case_bound(gpu_available):
    """All-positive operands at K = 4096: no cancellation, so rounding errors
    do not average out; the result must still satisfy the worst-case bound
    (K + 2) * 2^-24 that any fp32 summation order obeys."""
    g = torch.Generator().manual_seed(9)
    K = 4096
    A = torch.rand(64, K, generator=g)
    B = torch.rand(K, 64, generator=g)
    C0 = torch.rand(64, 64, generator=g)
    say("[positive] 64x64x4096")
    C, _, _ = run_gemm(A, B, C0, 1.0, 1.0)
    assert ratio(C, A, B, C0, 1.0, 1.0) <= (K + 2) * 2.0 ** -24


SPLIT_SHAPES = [(16, 8192, 8192), (1, 256, 1024), (7, 1000, 4100), (16, 136, 5000), (3, 4096, 2048),
                (16, 520, 1030), (12, 128, 1200)]


def test_split_k_skinny_exact_and_reusable_workspace(gpu_available):
    """The split-K path with one shared workspace: every row count 1..16 and
    ragged N and K, called back to back with different shapes (and so
    different split counts), must equal the oracle exactly each time.  The
    workspace starts out as NaN bytes: its contents on entry must not matter."""
    ws = tg.workspace(16, 8192, 8192)          # largest of the shapes below
    ws.fill_(0xFF)
    for i, (M, N, K) in enumerate(SPLIT_SHAPES + [(m, 640, 2304) for m in range(1, 17)]):
        assert tg.gemm_workspace_size(tg.GEMM_DTYPE_F32, M, N, K) <= ws.numel()
        A, B, C0 = make_integer_inputs(M, N, K, seed=200 + i)
        st, pl = tg.gemm_plan_query(tg.GEMM_DTYPE_F32, M, N, K, -1.0, 0x1000, K, 0x1000, N, 2.0, 0x1000, N, 0,
                                    ws.numel())
        assert pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK, (M, N, K, pl)
        say(f"[split-k] M={M} N={N} K={K} grid={pl['grid']} seed={200 + i}")
        C, _, _ = run_gemm(A, B, C0, -1.0, 2.0, ws=ws)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, -1.0, 2.0),
                                      err_msg=f"split-k {M}x{N}x{K}")


def test_split_k_skinny_deterministic(gpu_available):
    from tiled_gemm_f32_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS["f32_16x8192x8192"]
    A, B, C0 = make_inputs(w)
    Ad, Bd = A.cuda(), B.cuda()
    ws = tg.workspace(w.M, w.N, w.K)
    say("[split-k determinism] 16x8192x8192 x20")
    outs = [tg.gemm(Ad, Bd, ws=ws) for _ in range(20)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("tile", [64, 128])
@pytest.mark.parametrize("va", [1, 4])
def test_f32_ring_small_tiles_match_register_staged(gpu_available, va, tile):
    """The 64 x 64 and 128 x 128 fp32 rings (A loaded 4 or 16 bytes per lane)
    pair the same k in the same order as the register-staged kernels of
    their tile: on random data the two give the same bits, on integer data
    both equal the oracle.  K of 777, 255 and 1001 make A's rows unaligned
    (4-byte loads); K of 16, 17 and 3 are one slice, one slice and a bit, and
    part of one."""
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    ns = 6 if tile == 64 else 4
    ring = ids[f"f32_mfma32_{tile}x{tile}x16_w2x2_a{va}b4_ring{ns}"]
    staged = ids[f"f32_mfma32_{tile}x{tile}x16_w2x2_a{va}b4"]
    shapes = ([(1000, 3000, 777), (257, 264, 255), (65, 68, 17), (64, 64, 3), (130, 1028, 1001)] if va == 1 else
              [(1024, 1024, 1024), (256, 256, 256), (65, 68, 16), (300, 520, 1032), (64, 4, 4)])
    for M, N, K in shapes:
        st, _ = tg.gemm_plan_query(tg.GEMM_DTYPE_F32, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.0, 0x1000, N, ring, 0)
        assert st == tg.GEMM_OK, (M, N, K)
        A, B, C0 = make_random_inputs(M, N, K, seed=M + 3 * N + K, dist="uniform")
        say(f"[f32 ring {tile} a{va}] random M={M} N={N} K={K}")
        C1, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=ring)
        C2, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=staged)
        np.testing.assert_array_equal(C1, C2, err_msg=f"{M}x{N}x{K}")
        assert ratio(C1, A, B, C0, 2.0, -1.0) <= TOL["f32"]
        Ai, Bi, Ci = make_integer_inputs(M, N, K, seed=M * 5 + K)
        say(f"[f32 ring {tile} a{va}] exact M={M} N={N} K={K}")
        for alpha, beta in [(2.0, -1.0), (1.0, 0.0)]:
            C, _, _ = run_gemm(Ai, Bi, Ci, alpha, beta, kernel=ring)
            np.testing.assert_array_equal(C.astype(np.float64), _exact(Ai, Bi, Ci, alpha, beta),
                                          err_msg=f"{M}x{N}x{K}")


@pytest.mark.parametrize("tile", [64, 128])
@pytest.mark.parametrize("layout", ["nt", "tn", "tt"])
def test_f32_ring_small_tiles_transposed_layouts(gpu_available, layout, tile):
    """The 64 x 64 and 128 x 128 fp32 rings with A stored K x M and/or B stored
    N x K: on random data the same bits as the register-staged untransposed
    kernel of the tile on the untransposed operands (same operand order and
    k order per lane), on integer data the oracle's bits.  N is free when B
    is stored N x K (ragged N below)."""
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    ns = 6 if tile == 64 else 4
    ring = ids[f"f32_mfma32_{tile}x{tile}x16_w2x2_a4b4_{layout}_ring{ns}"]
    staged = ids[f"f32_mfma32_{tile}x{tile}x16_w2x2_a4b4"]
    op_a, op_b = layout[0].upper(), layout[1].upper()
    for M, N, K, n_free in [(1024, 1024, 1024, 0), (260, 264, 68, 3), (64, 68, 4, 0), (300, 520, 1032, 1),
                            (132, 8, 16, 1)]:
        if op_b == "T":
            N += n_free                                 # B stored N x K leaves N free
        A, B, C0 = make_random_inputs(M, N, K, seed=M + 5 * N + K, dist="uniform")
        As = A.t().contiguous() if op_a == "T" else A
        Bs = B.t().contiguous() if op_b == "T" else B
        say(f"[f32 ring {tile} {layout}] random M={M} N={N} K={K}")
        C1, _, _ = run_gemm(As, Bs, C0, 2.0, -1.0, kernel=ring, op_a=op_a, op_b=op_b)
        if N % 4 == 0:
            C2, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=staged)
            np.testing.assert_array_equal(C1, C2, err_msg=f"{M}x{N}x{K}")
        assert ratio(C1, A, B, C0, 2.0, -1.0) <= TOL["f32"]
        Ai, Bi, Ci = make_integer_inputs(M, N, K, seed=M * 3 + K)
        Ais = Ai.t().contiguous() if op_a == "T" else Ai
        Bis = Bi.t().contiguous() if op_b == "T" else Bi
        say(f"[f32 ring {tile} {layout}] exact M={M} N={N} K={K}")
        C, _, _ = run_gemm(Ais, Bis, Ci, 2.0, -1.0, kernel=ring, op_a=op_a, op_b=op_b)
        np.testing.assert_array_equal(C.astype(np.float64), _exact(Ai, Bi, Ci, 2.0, -1.0), err_msg=f"{M}x{N}x{K}")
