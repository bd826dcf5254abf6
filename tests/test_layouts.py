"""GPU parity of gemm_general: transposed operand layouts for every operand
type, and fp8 (OCP E4M3) operands.

Transposed operands are the stored transposes of seeded M x K / K x N
draws; the oracle multiplies the transposes of what it is given.

Tolerances:
* fp32 and bf16: the error ratio of the untransposed paths (2e-6, 1e-5).
* fp8, every kernel:
      |C - ref| <= 7 * 2^-13 * G + (2e-6 + 2^-24) * D
  G is the oracle's group-maximum sum (|alpha| times, over each run of 8
  consecutive k, the largest |product|) and D the error-ratio denominator.
  The fp8 matrix instruction sums each run of 8 products after truncating
  them below 2^-13 of the run's largest power of two (measured on gfx950
  with in-bounds probes), so each of the other 7 products of a run loses
  less than 2^-13 of the run maximum; runs, slices and C0 are then added in
  fp32, bounded like the fp32 path.  The general kernel multiplies fp8
  values exactly in fp32 and meets the same bound with room to spare.
* Integer operands (|v| <= 4) give exact products, exact run sums (the
  smallest nonzero product is at most 4 bits below the largest) and sums
  below 2^24, so every kernel must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, run_gemm, say

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
U32 = 2.0 ** -24
RUN_TRUNC = 7 * 2.0 ** -13
FP8_RING = "fp8_mfma32_256x256x64_w2x2_nt_ring4"
BF16_NT_RING = "bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4"
BF16_TN_RING = "bf16_mfma32_256x256x32_w2x2_a8b8_tn_ring4"
BF16_TT_RING = "bf16_mfma32_256x256x32_w2x2_a8b8_tt_ring4"
FP8_NN_RING = "fp8_mfma32_256x256x64_w2x2_nn_ring4"
FP8_TN_RING = "fp8_mfma32_256x256x64_w2x2_tn_ring4"
FP8_TT_RING = "fp8_mfma32_256x256x64_w2x2_tt_ring4"
F32_NT_RING = "f32_mfma32_256x256x16_w2x2_a4b4_nt_ring4"
F32_TN_RING = "f32_mfma32_256x256x16_w2x2_a4b4_tn_ring4"
F32_TT_RING = "f32_mfma32_256x256x16_w2x2_a4b4_tt_ring4"
# (dtype, kernel, op_a, op_b) of every ring kernel for a transposed layout
T_RINGS = [("fp8f32", FP8_RING, "N", "T"), ("bf16f32", BF16_NT_RING, "N", "T"),
           ("bf16f32", BF16_TN_RING, "T", "N"), ("bf16f32", BF16_TT_RING, "T", "T"),
           ("f32", F32_NT_RING, "N", "T"), ("f32", F32_TN_RING, "T", "N"), ("f32", F32_TT_RING, "T", "T"),
           ("fp8f32", FP8_NN_RING, "N", "N"), ("fp8f32", FP8_TN_RING, "T", "N"), ("fp8f32", FP8_TT_RING, "T", "T")]


def stored(A, B, op_a, op_b):
    """The operands as stored for the layout: transposed copies where asked."""
    return (A.t().contiguous() if op_a == "T" else A), (B.t().contiguous() if op_b == "T" else B)


def ref_of(As, Bs, C0, alpha, beta, op_a, op_b):
    return oracle.gemm_ref(host_view(As), host_view(Bs), alpha, beta, C0.numpy(), op_a, op_b)


def check(C, As, Bs, C0, alpha, beta, op_a, op_b, dtype, bias=None, act="none"):
    """Assert the tolerance above; returns the worst err / allowance."""
    a, b, c0 = host_view(As), host_view(Bs), C0.numpy()
    bias_np = bias.numpy() if bias is not None else None
    ref = oracle.gemm_epilogue_ref(a, b, alpha, beta, c0, bias_np, act, op_a, op_b)
    D = oracle.gemm_absbound(a, b, alpha, beta, c0, op_a, op_b)
    if bias_np is not None:
        D = D + np.abs(bias_np.astype(np.float64))
    if dtype == "fp8f32":
        allow = RUN_TRUNC * oracle.gemm_groupmax(a, b, alpha, op_a, op_b) + (2e-6 + U32) * D
    else:
        allow = TOL[dtype] * D
    if act == "gelu":
        z = oracle.gemm_epilogue_ref(a, b, alpha, beta, c0, bias_np, "none", op_a, op_b)
        allow = 1.13 * allow + 6e-7 * np.abs(z)
    err = np.abs(np.asarray(C, np.float64) - ref)
    assert np.all(np.isfinite(err)), "non-finite difference"
    bad = err > allow
    assert not np.any(bad), f"{int(bad.sum())} elements out of bound; worst excess {float(np.max(err - allow)):.3e}"
    nz = allow > 0
    return float(np.max(err[nz] / allow[nz])) if np.any(nz) else 0.0


def kernels_for(dtype, op_a, op_b):
    bit = 2 * (op_a == "T") + (op_b == "T")
    return [k for k in tg.kernels() if k["dtype"] == DT[dtype] and (k["layouts"] >> bit) & 1
            and k["path"] == tg.GEMM_PATH_TILED]


def runnable(dtype, op_a, op_b, M, N, K, kid, ws_bytes=0):
    lda = K if op_a == "N" else M
    ldb = N if op_b == "N" else K
    st, pl = tg.gemm_plan_query_general(DT[dtype], 0 if op_a == "N" else 1, 0 if op_b == "N" else 1, M, N, K, 1.0,
                                        0x1000, lda, 0x1000, ldb, 0.5, 0x1000, N, kid, ws_bytes)
    return st == tg.GEMM_OK, pl


@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_every_kernel_every_layout_exact(gpu_available, dtype, ops):
    """Integer data through every kernel that runs the layout: bit-exact."""
    op_a, op_b = ops
    M, N, K = 300, 264, 208          # ragged tiles; K a multiple of 16 so the fp8 ring runs too
    A, B, C0 = make_integer_inputs(M, N, K, seed=700, dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    ref = ref_of(As, Bs, C0, 2.0, -1.0, op_a, op_b)
    ran = 0
    for k in kernels_for(dtype, op_a, op_b):
        ok, _ = runnable(dtype, op_a, op_b, M, N, K, k["id"])
        if not ok:
            continue
        say(f"[layout exact] {dtype} op_a={op_a} op_b={op_b} kernel={k['name']} M={M} N={N} K={K} seed=700")
        C, _, _ = run_gemm(As, Bs, C0, 2.0, -1.0, kernel=k["id"], op_a=op_a, op_b=op_b)
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=k["name"])
        ran += 1
    assert ran >= 1


@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_every_kernel_every_layout_random(gpu_available, dtype, ops):
    op_a, op_b = ops
    M, N, K = 520, 390, 1040
    A, B, C0 = make_random_inputs(M, N, K, seed=701, dist="normal", dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    for k in kernels_for(dtype, op_a, op_b):
        ok, _ = runnable(dtype, op_a, op_b, M, N, K, k["id"])
        if not ok:
            continue
        say(f"[layout random] {dtype} op_a={op_a} op_b={op_b} kernel={k['name']} M={M} N={N} K={K} seed=701")
        C, _, _ = run_gemm(As, Bs, C0, 0.75, 0.5, kernel=k["id"], op_a=op_a, op_b=op_b)
        r = check(C, As, Bs, C0, 0.75, 0.5, op_a, op_b, dtype)
        say(f"[layout random] worst err/allowance {r:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
@pytest.mark.parametrize("ops", [("N", "T"), ("T", "N"), ("T", "T")], ids=lambda o: o[0] + o[1])
def test_padded_and_unaligned_transposed(gpu_available, dtype, ops):
    """Transposed operands inside padded buffers (NaN padding), bases one
    element off alignment, C padded: the library's own choice."""
    op_a, op_b = ops
    M, N, K = 130, 70, 90
    A, B, C0 = make_integer_inputs(M, N, K, seed=702, dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    say(f"[layout padded] {dtype} op_a={op_a} op_b={op_b} M={M} N={N} K={K} pad=(3,5,2) offset=(1,1,0)")
    C, _, _ = run_gemm(As, Bs, C0, 1.0, 1.0, pad=(3, 5, 2), offset=(1, 1, 0), op_a=op_a, op_b=op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, 1.0, 1.0, op_a, op_b))


@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: o[0] + o[1])
def test_k_split_every_layout(gpu_available, dtype, ops):
    """The tiled K split rebases k along rows or down columns by layout."""
    op_a, op_b = ops
    M, N, K = 256, 512, 6000
    ws = tg.workspace(M, N, K, dtype=DT[dtype])
    ws.fill_(0xFF)
    A, B, C0 = make_integer_inputs(M, N, K, seed=703, dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    ok, pl = runnable(dtype, op_a, op_b, M, N, K, 0, ws.numel())
    assert ok and pl["splits"] > 1, pl
    say(f"[layout k-split] {dtype} op_a={op_a} op_b={op_b} M={M} N={N} K={K} splits={pl['splits']} "
        f"kernel={tg.gemm_kernel_query(pl['kernel_id'])['name']}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0, 0.5, ws=ws, op_a=op_a, op_b=op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, 1.0, 0.5, op_a, op_b))


# ----------------------------------------------------------------------------- the A x B^T ring kernels

FP8_SHAPES = [
    (256, 256, 64),        # one tile, one slice
    (1000, 1001, 1040),    # ragged M and N (N not a multiple of 4), a partial last slice
    (33, 2048, 4096),      # thin M
    (2048, 40, 2048),      # thin N
    (1024, 1024, 16),      # K smaller than one slice
]


def ring_shape(shape, op_a, op_b, dtype="bf16f32"):
    """Adjust an edge shape to what a ring kernel for this layout needs: the
    stored rows of A and B are whole 16-byte chunks (M is A^T's row length,
    N is an untransposed B's; 16 fp8 or 8 wider elements)."""
    M, N, K = shape
    step = 16 if dtype == "fp8f32" else 8
    if op_a == "T":
        M = -(-M // step) * step
    if op_b == "N":
        N = -(-N // step) * step
    return M, N, K


@pytest.mark.parametrize("ring_case", T_RINGS, ids=lambda c: c[1])
@pytest.mark.parametrize("shape", FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_transposed_ring_shapes(gpu_available, ring_case, shape):
    """The ring kernels for transposed layouts, forced (small problems would
    otherwise take the smallest tile), on edge shapes."""
    dtype, ring_name, op_a, op_b = ring_case
    M, N, K = ring_shape(shape, op_a, op_b, dtype)
    ring = [k["id"] for k in tg.kernels() if k["name"] == ring_name][0]
    ok, _ = runnable(dtype, op_a, op_b, M, N, K, ring)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=710, dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    say(f"[t ring] {ring_name} exact M={M} N={N} K={K} seed=710")
    C, _, _ = run_gemm(As, Bs, C0, -1.0, 2.0, kernel=ring, op_a=op_a, op_b=op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, -1.0, 2.0, op_a, op_b))
    A, B, C0 = make_random_inputs(M, N, K, seed=711, dist="normal", dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    say(f"[t ring] {ring_name} random M={M} N={N} K={K} seed=711")
    C, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=ring, op_a=op_a, op_b=op_b)
    r = check(C, As, Bs, C0, 0.5, 0.25, op_a, op_b, dtype)
    say(f"[t ring] worst err/allowance {r:.3e}")


@pytest.mark.parametrize("ring_case", T_RINGS, ids=lambda c: c[1])
@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("c_offset", [0, 1])
def test_transposed_ring_epilogue_and_c_alignment(gpu_available, ring_case, act, c_offset):
    dtype, ring_name, op_a, op_b = ring_case
    M, N, K = ring_shape((520, 777, 512), op_a, op_b, dtype)
    A, B, C0 = make_random_inputs(M, N, K, seed=712, dist="normal", dtype=dtype)
    As, Bs = stored(A, B, op_a, op_b)
    bias = make_bias(N, seed=713)
    alpha = 1.0 / np.sqrt(K)
    ring = [k["id"] for k in tg.kernels() if k["name"] == ring_name][0]
    say(f"[t ring] {ring_name} epilogue act={act} M={M} N={N} K={K} c_offset={c_offset}")
    C, _, _ = run_gemm(As, Bs, C0, alpha, -0.5, kernel=ring, offset=(0, 0, c_offset), bias=bias, activation=act,
                       op_a=op_a, op_b=op_b)
    check(C, As, Bs, C0, alpha, -0.5, op_a, op_b, dtype, bias=bias, act=act)


NT_LINES = "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines"
NT_LINES_SHAPES = [
    (256, 256, 1024),      # one tile
    (1000, 1001, 1040),    # ragged M and N (runs of 4 columns straddle N), a partial last slice
    (33, 2048, 4096),      # thin M
    (2048, 40, 2048),      # thin N
    (4100, 4300, 1096),    # more tiles than compute units, ragged last tiles
]


@pytest.mark.parametrize("shape", NT_LINES_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nt_lines_kernel(gpu_available, shape):
    """The whole-line bf16 kernel with B stored N x K, forced: exact on
    integer data, and on random data the same bits as the B-transposed ring
    kernel (the same k pairing and summation order per lane)."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    lines, ring = ids[NT_LINES], ids[BF16_NT_RING]
    ok, _ = runnable("bf16f32", "N", "T", M, N, K, lines)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=720, dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[nt lines] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=720")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=lines, op_a="N", op_b="T")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "N", "T"))
    A, B, C0 = make_random_inputs(M, N, K, seed=721, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    say(f"[nt lines] random M={M} N={N} K={K} seed=721, against the ring")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=lines, op_a="N", op_b="T")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=ring, op_a="N", op_b="T")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "N", "T", "bf16f32")


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("c_offset", [0, 1])
def test_nt_lines_epilogue_and_c_alignment(gpu_available, act, c_offset):
    M, N, K = 520, 777, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=722, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    bias = make_bias(N, seed=723)
    lines = [k["id"] for k in tg.kernels() if k["name"] == NT_LINES][0]
    say(f"[nt lines] epilogue act={act} M={M} N={N} K={K} c_offset={c_offset}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0 / np.sqrt(K), -0.5, kernel=lines, offset=(0, 0, c_offset), bias=bias,
                       activation=act, op_a="N", op_b="T")
    check(C, As, Bs, C0, 1.0 / np.sqrt(K), -0.5, "N", "T", "bf16f32", bias=bias, act=act)


TN_LINES = "bf16_mfma32_256x256x32_w2x2_a8b8_tn_lines"


@pytest.mark.parametrize("shape", [(256, 256, 1024), (1000, 1000, 1040), (40, 2048, 4096), (2048, 40, 2048),
                                   (4104, 4296, 1096), (264, 136, 48)], ids=lambda s: "x".join(map(str, s)))
def test_tn_lines_kernel(gpu_available, shape):
    """The whole-line bf16 kernel with A stored K x M, forced: exact on
    integer data (with beta on and off; K of 48 is one slice and a half),
    and on random data the same bits as the A-transposed ring kernel."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    lines, ring = ids[TN_LINES], ids[BF16_TN_RING]
    ok, _ = runnable("bf16f32", "T", "N", M, N, K, lines)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=750, dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[tn lines] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=750")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=lines, op_a="T", op_b="N")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "T", "N"))
    A, B, C0 = make_random_inputs(M, N, K, seed=751, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    say(f"[tn lines] random M={M} N={N} K={K} seed=751, against the ring")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=lines, op_a="T", op_b="N")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=ring, op_a="T", op_b="N")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "T", "N", "bf16f32")


def test_tn_lines_epilogue_padded(gpu_available):
    """Bias and GELU with A^T, B and C inside NaN-padded rows (padding 8, 24
    and 3 elements: A^T's padding reaches only rows of C that are never
    written)."""
    M, N, K = 520, 776, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=752, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    bias = make_bias(N, seed=753)
    lines = [k["id"] for k in tg.kernels() if k["name"] == TN_LINES][0]
    say(f"[tn lines] epilogue gelu, padded, M={M} N={N} K={K}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0 / np.sqrt(K), -0.5, kernel=lines, pad=(8, 24, 3), bias=bias,
                       activation="gelu", op_a="T", op_b="N")
    check(C, As, Bs, C0, 1.0 / np.sqrt(K), -0.5, "T", "N", "bf16f32", bias=bias, act="gelu")


TN_LINES128 = "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines"


@pytest.mark.parametrize("shape", [(128, 128, 256), (1000, 1000, 1040), (40, 2048, 4096), (2048, 40, 2048),
                                   (2104, 2056, 1096), (264, 136, 48), (136, 264, 32), (136, 128, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_tn_lines128_kernel(gpu_available, shape):
    """The 128 x 128 whole-line kernel with A stored K x M, forced: exact on
    integer data (K of 8, 32 and 48), and on random data the same bits as
    the 256 x 256 one."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    small, big = ids[TN_LINES128], ids[TN_LINES]
    ok, _ = runnable("bf16f32", "T", "N", M, N, K, small)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=768, dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[tn lines128] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=768")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=small, op_a="T", op_b="N")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "T", "N"))
    A, B, C0 = make_random_inputs(M, N, K, seed=769, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    say(f"[tn lines128] random M={M} N={N} K={K} seed=769, against the 256 x 256 kernel")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=small, op_a="T", op_b="N")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=big, op_a="T", op_b="N")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "T", "N", "bf16f32")


def test_tn_lines128_epilogue_padded(gpu_available):
    """Bias and GELU with A^T, B and C inside NaN-padded rows (padding 8, 24
    and 3 elements)."""
    M, N, K = 520, 776, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=770, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "T", "N")
    bias = make_bias(N, seed=771)
    kid = [k["id"] for k in tg.kernels() if k["name"] == TN_LINES128][0]
    say(f"[tn lines128] epilogue gelu, padded, M={M} N={N} K={K}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0 / np.sqrt(K), -0.5, kernel=kid, pad=(8, 24, 3), bias=bias,
                       activation="gelu", op_a="T", op_b="N")
    check(C, As, Bs, C0, 1.0 / np.sqrt(K), -0.5, "T", "N", "bf16f32", bias=bias, act="gelu")


FP8_LINES = "fp8_mfma32_256x256x128_w2x2_nt_lines"


@pytest.mark.parametrize("shape", [(256, 256, 1024), (1000, 1001, 1040), (33, 2048, 4096), (2048, 40, 2048),
                                   (4100, 4300, 1088), (300, 264, 80)], ids=lambda s: "x".join(map(str, s)))
def test_fp8_lines_kernel(gpu_available, shape):
    """The whole-line fp8 kernel (B stored N x K), forced: exact on integer
    data (K of 80 is one whole pair and a partial one), and on random data
    the same bits as the fp8 ring (the same byte pairing and run order)."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    lines, ring = ids[FP8_LINES], ids[FP8_RING]
    ok, _ = runnable("fp8f32", "N", "T", M, N, K, lines)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=740, dtype="fp8f32")
    As, Bs = stored(A, B, "N", "T")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[fp8 lines] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=740")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=lines, op_a="N", op_b="T")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "N", "T"))
    A, B, C0 = make_random_inputs(M, N, K, seed=741, dist="normal", dtype="fp8f32")
    As, Bs = stored(A, B, "N", "T")
    say(f"[fp8 lines] random M={M} N={N} K={K} seed=741, against the ring")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=lines, op_a="N", op_b="T")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=ring, op_a="N", op_b="T")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "N", "T", "fp8f32")


FP8_LINES128 = "fp8_mfma32_128x128x128_w2x2_nt_lines"


@pytest.mark.parametrize("shape", [(128, 128, 256), (1000, 1001, 1040), (33, 2048, 4096), (2048, 40, 2048),
                                   (2100, 2059, 1088), (300, 264, 80), (136, 130, 64), (130, 136, 16)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_lines128_kernel(gpu_available, shape):
    """The 128 x 128 whole-line fp8 kernel, forced: exact on integer data
    (K of 16, 64 and 80: part of a slice, one slice, a pair and a part), and
    on random data the same bits as the 256 x 256 one."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    small, big = ids[FP8_LINES128], ids[FP8_LINES]
    ok, _ = runnable("fp8f32", "N", "T", M, N, K, small)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=772, dtype="fp8f32")
    As, Bs = stored(A, B, "N", "T")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[fp8 lines128] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=772")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=small, op_a="N", op_b="T")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "N", "T"))
    A, B, C0 = make_random_inputs(M, N, K, seed=773, dist="normal", dtype="fp8f32")
    As, Bs = stored(A, B, "N", "T")
    say(f"[fp8 lines128] random M={M} N={N} K={K} seed=773, against the 256 x 256 kernel")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=small, op_a="N", op_b="T")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=big, op_a="N", op_b="T")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "N", "T", "fp8f32")


FP8_RING128 = {("N", "N"): ("fp8_mfma32_128x128x64_w2x2_nn_ring4", FP8_NN_RING),
               ("T", "N"): ("fp8_mfma32_128x128x64_w2x2_tn_ring4", FP8_TN_RING),
               ("T", "T"): ("fp8_mfma32_128x128x64_w2x2_tt_ring4", FP8_TT_RING)}


@pytest.mark.parametrize("ops", list(FP8_RING128), ids=lambda o: o[0] + o[1])
@pytest.mark.parametrize("shape", [(128, 128, 256), (1008, 1024, 1040), (48, 2048, 4096), (2048, 48, 2048),
                                   (2096, 2064, 1088), (304, 272, 80), (144, 128, 64), (128, 144, 16)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_ring128(gpu_available, ops, shape):
    """The 128 x 128 fp8 rings (A stored K x M and/or B stored K x N), forced:
    exact on integer data (K of 16, 64 and 80), and on random data the same
    bits as the 256 x 256 ring of the layout (the same byte pairing and slice
    order)."""
    op_a, op_b = ops
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    small, big = (ids[n] for n in FP8_RING128[ops])
    ok, _ = runnable("fp8f32", op_a, op_b, M, N, K, small)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=774, dtype="fp8f32")
    As, Bs = stored(A, B, op_a, op_b)
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[fp8 ring128 {op_a}{op_b}] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=774")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=small, op_a=op_a, op_b=op_b)
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, op_a, op_b))
    A, B, C0 = make_random_inputs(M, N, K, seed=775, dist="normal", dtype="fp8f32")
    As, Bs = stored(A, B, op_a, op_b)
    say(f"[fp8 ring128 {op_a}{op_b}] random M={M} N={N} K={K} seed=775, against the 256 x 256 ring")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=small, op_a=op_a, op_b=op_b)
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=big, op_a=op_a, op_b=op_b)
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, op_a, op_b, "fp8f32")


@pytest.mark.parametrize("name", [FP8_LINES, FP8_LINES128])
def test_fp8_lines_epilogue_padded(gpu_available, name):
    """Bias and GELU with A, B and C inside NaN-padded rows (padding 16, 48
    and 3 elements), ragged N."""
    M, N, K = 520, 777, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=742, dist="normal", dtype="fp8f32")
    As, Bs = stored(A, B, "N", "T")
    bias = make_bias(N, seed=743)
    lines = [k["id"] for k in tg.kernels() if k["name"] == name][0]
    say(f"[fp8 lines] {name} epilogue gelu, padded, M={M} N={N} K={K}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0 / np.sqrt(K), -0.5, kernel=lines, pad=(16, 48, 3), bias=bias,
                       activation="gelu", op_a="N", op_b="T")
    check(C, As, Bs, C0, 1.0 / np.sqrt(K), -0.5, "N", "T", "fp8f32", bias=bias, act="gelu")


NN_LINES = "bf16_mfma32_256x256x64_w2x2_a8b8_lines"
NN_LINES128 = "bf16_mfma32_128x128x64_w2x2_a8b8_lines"


@pytest.mark.parametrize("shape", [(128, 128, 256), (1000, 1000, 1040), (40, 2048, 4096), (2048, 40, 2048),
                                   (2100, 2056, 1096), (264, 136, 48), (136, 264, 32), (130, 136, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_lines128_kernel(gpu_available, shape):
    """The 128 x 128 whole-line bf16 kernel, forced: exact on integer data
    (K of 8, 32 and 48: part of a slice, one slice, a slice and a half), and
    on random data the same bits as the 256 x 256 whole-line kernel (the same
    k pairing and summation order per lane)."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    small, big = ids[NN_LINES128], ids[NN_LINES]
    ok, _ = runnable("bf16f32", "N", "N", M, N, K, small)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=760, dtype="bf16f32")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[lines128] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=760")
        C, _, _ = run_gemm(A, B, C0, alpha, beta, kernel=small)
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(A, B, C0, alpha, beta, "N", "N"))
    A, B, C0 = make_random_inputs(M, N, K, seed=761, dist="normal", dtype="bf16f32")
    say(f"[lines128] random M={M} N={N} K={K} seed=761, against the 256 x 256 kernel")
    C1, _, _ = run_gemm(A, B, C0, 0.5, 0.25, kernel=small)
    C2, _, _ = run_gemm(A, B, C0, 0.5, 0.25, kernel=big)
    np.testing.assert_array_equal(C1, C2)
    check(C1, A, B, C0, 0.5, 0.25, "N", "N", "bf16f32")


NT_LINES128 = "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines"


@pytest.mark.parametrize("shape", [(128, 128, 256), (1000, 1001, 1040), (40, 2048, 4096), (2048, 41, 2048),
                                   (2100, 2059, 1096), (264, 133, 48), (136, 264, 32), (130, 131, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nt_lines128_kernel(gpu_available, shape):
    """The 128 x 128 whole-line kernel with B stored N x K, forced: exact on
    integer data (ragged N: runs of 4 columns straddle it; K of 8, 32 and
    48), and on random data the same bits as the 256 x 256 one."""
    M, N, K = shape
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    small, big = ids[NT_LINES128], ids[NT_LINES]
    ok, _ = runnable("bf16f32", "N", "T", M, N, K, small)
    assert ok
    A, B, C0 = make_integer_inputs(M, N, K, seed=764, dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    for alpha, beta in [(-1.0, 2.0), (1.0, 0.0)]:
        say(f"[nt lines128] exact M={M} N={N} K={K} alpha={alpha} beta={beta} seed=764")
        C, _, _ = run_gemm(As, Bs, C0, alpha, beta, kernel=small, op_a="N", op_b="T")
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, alpha, beta, "N", "T"))
    A, B, C0 = make_random_inputs(M, N, K, seed=765, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    say(f"[nt lines128] random M={M} N={N} K={K} seed=765, against the 256 x 256 kernel")
    C1, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=small, op_a="N", op_b="T")
    C2, _, _ = run_gemm(As, Bs, C0, 0.5, 0.25, kernel=big, op_a="N", op_b="T")
    np.testing.assert_array_equal(C1, C2)
    check(C1, As, Bs, C0, 0.5, 0.25, "N", "T", "bf16f32")


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("c_offset", [0, 1])
def test_nt_lines128_epilogue_and_c_alignment(gpu_available, act, c_offset):
    M, N, K = 520, 777, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=766, dist="normal", dtype="bf16f32")
    As, Bs = stored(A, B, "N", "T")
    bias = make_bias(N, seed=767)
    kid = [k["id"] for k in tg.kernels() if k["name"] == NT_LINES128][0]
    say(f"[nt lines128] epilogue act={act} M={M} N={N} K={K} c_offset={c_offset}")
    C, _, _ = run_gemm(As, Bs, C0, 1.0 / np.sqrt(K), -0.5, kernel=kid, offset=(0, 0, c_offset), bias=bias,
                       activation=act, op_a="N", op_b="T")
    check(C, As, Bs, C0, 1.0 / np.sqrt(K), -0.5, "N", "T", "bf16f32", bias=bias, act=act)


@pytest.mark.parametrize("act", ["relu", "gelu"])
@pytest.mark.parametrize("c_offset", [0, 1])
def test_lines128_epilogue_and_c_alignment(gpu_available, act, c_offset):
    M, N, K = 520, 776, 1024
    A, B, C0 = make_random_inputs(M, N, K, seed=762, dist="normal", dtype="bf16f32")
    bias = make_bias(N, seed=763)
    kid = [k["id"] for k in tg.kernels() if k["name"] == NN_LINES128][0]
    say(f"[lines128] epilogue act={act} M={M} N={N} K={K} c_offset={c_offset}")
    C, _, _ = run_gemm(A, B, C0, 1.0 / np.sqrt(K), -0.5, kernel=kid, offset=(0, 0, c_offset), bias=bias,
                       activation=act)
    check(C, A, B, C0, 1.0 / np.sqrt(K), -0.5, "N", "N", "bf16f32", bias=bias, act=act)


@pytest.mark.parametrize("name", [NN_LINES, NT_LINES, NN_LINES128, NT_LINES128])
def test_lines_kernels_padded_operands(gpu_available, name):
    """The whole-line kernels on operands inside wider buffers: A, B and C
    padded by 8, 24 and 5 elements per row, the padding NaN (it must never
    reach C), ragged M, N and K; integer data, so the result is exact."""
    op_b = "T" if name in (NT_LINES, NT_LINES128) else "N"
    kid = [k["id"] for k in tg.kernels() if k["name"] == name][0]
    for M, N, K in [(300, 520 if op_b == "N" else 517, 1096), (1030, 264, 2056)]:
        A, B, C0 = make_integer_inputs(M, N, K, seed=730 + M, dtype="bf16f32")
        As, Bs = stored(A, B, "N", op_b)
        say(f"[lines padded] {name} M={M} N={N} K={K} pad=(8, 24, 5)")
        C, _, _ = run_gemm(As, Bs, C0, 2.0, -1.0, kernel=kid, pad=(8, 24, 5), op_a="N", op_b=op_b)
        np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, 2.0, -1.0, "N", op_b))


def test_nt_lines_is_the_choice_for_weights_stored_n_by_k():
    """bf16 A x B^T with K >= 1024 and whole 16-byte rows goes to the
    whole-line kernel; K below 1024 stays on the ring."""
    st, pl = tg.gemm_plan_query_general(DT["bf16f32"], 0, 1, 8192, 8192, 8192, 1.0, 0x1000, 8192, 0x1000, 8192,
                                        0.0, 0x1000, 8192, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] == NT_LINES
    st, pl = tg.gemm_plan_query_general(DT["bf16f32"], 0, 1, 8192, 8192, 512, 1.0, 0x1000, 512, 0x1000, 512,
                                        0.0, 0x1000, 8192, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] != NT_LINES


def test_fp8_ring_deterministic_and_bench_shape_sampled(gpu_available):
    """fp8 8192^3 (A x B^T): integer data exact on sampled rows and columns,
    normal data within the bound; 5 calls give the same bits."""
    n = 8192
    A, B, C0 = make_integer_inputs(n, n, n, seed=714, dtype="fp8f32")
    Bt = B.t().contiguous()
    Ad = A.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    Bd = Bt.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    say(f"[fp8 ring] {n}^3 exact sampled, x5 determinism")
    outs = [tg.gemm(Ad, Bd, op_b="T") for _ in range(5)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    C = outs[0].cpu().numpy()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 255, 256, n - 1]) | set(rng.integers(0, n, 6).tolist()))
    cols = sorted(set([0, 255, 256, n - 1]) | set(rng.integers(0, n, 6).tolist()))
    a, bt = host_view(A), host_view(Bt)
    np.testing.assert_array_equal(C[rows].astype(np.float64), oracle.gemm_ref(a[rows], bt, op_b="T"))
    np.testing.assert_array_equal(C[:, cols].astype(np.float64),
                                  oracle.gemm_ref(a, np.ascontiguousarray(bt[cols]), op_b="T"))
    A, B, C0 = make_random_inputs(n, n, n, seed=715, dist="normal", dtype="fp8f32")
    Bt = B.t().contiguous()
    Ad = A.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    Bd = Bt.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    say(f"[fp8 ring] {n}^3 normal sampled")
    C = tg.gemm(Ad, Bd, op_b="T").cpu().numpy()
    zero = torch.zeros(len(rows), n)
    check(C[rows], A[rows], Bt, zero, 1.0, 0.0, "N", "T", "fp8f32")
    check(C[:, cols], A, Bt[cols].contiguous(), torch.zeros(n, len(cols)), 1.0, 0.0, "N", "T", "fp8f32")


# ----------------------------------------------------------------------------- decode with A stored K x M

F32_AT_SKINNY = ["f32_skinny_mfma16_n2_at_w8_u4", "f32_skinny_splitk_n128_at_w8_u1"]


@pytest.mark.parametrize("M", [1, 7, 16])
@pytest.mark.parametrize("NK", [(8192, 4096), (1000, 777), (40, 12288)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_skinny_a_transposed_exact(gpu_available, M, NK):
    """fp32, M <= 16, A stored K x M: both streaming kernels forced, and the
    library's choice with and without a workspace, bit-exact on integer data
    with bias and ReLU; A's leading dimension padded past M once."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=760 + M, dtype="f32")
    As = A.t().contiguous()
    bias = make_bias(N, seed=761, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu", "T", "N")
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_F32)
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    runs = [(n, ids[n], ws, (0, 0, 0)) for n in F32_AT_SKINNY] + [("auto", 0, None, (0, 0, 0)),
                                                                   ("auto ws", 0, ws, (0, 0, 0)),
                                                                   ("auto ws lda+5", 0, ws, (5, 0, 0))]
    for name, kid, w, pad in runs:
        say(f"[A^T skinny] {name} M={M} N={N} K={K} pad={pad[0]} seed={760 + M}")
        C, _, _ = run_gemm(As, B, C0, 2.0, -1.0, kernel=kid, ws=w, bias=bias, activation="relu", op_a="T",
                           pad=pad)
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)
    # (M = 1 with lda = 1 is the same memory as A stored 1 x K, and runs as that.)
    st, pl = tg.gemm_plan_query_general(tg.GEMM_DTYPE_F32, 1, 0, M, N, K, 1.0, 0x1000, max(M, 2), 0x1000, N, 0.0,
                                        0x1000, N, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] in F32_AT_SKINNY


@pytest.mark.parametrize("with_ws", [False, True], ids=["no_ws", "ws"])
def test_skinny_a_transposed_random_full_size(gpu_available, with_ws):
    """16 x 8192 x 8192 with A stored K x M on U[-1,1] data (the decode
    workload's distribution): the fp32 error ratio, and the same bits as
    the call with A stored M x K on the same values."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=3, dist="uniform")
    As = A.t().contiguous()
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_F32) if with_ws else None
    say(f"[A^T skinny] auto M={M} N={N} K={K} uniform seed=3 ws={with_ws}")
    C, _, _ = run_gemm(As, B, C0, 1.0, 0.0, ws=ws, op_a="T")
    ref = oracle.gemm_ref(host_view(As), host_view(B), 1.0, 0.0, C0.numpy(), "T", "N")
    D = oracle.gemm_absbound(host_view(As), host_view(B), 1.0, 0.0, C0.numpy(), "T", "N")
    r = oracle.error_ratio(C, ref, D)
    say(f"[A^T skinny] ratio {r:.3e}")
    assert r <= TOL["f32"]
    # Same k pairing and summation order as the untransposed kernel of the same shape.
    C2, _, _ = run_gemm(A, B, C0, 1.0, 0.0, ws=ws)
    np.testing.assert_array_equal(C, C2)


BF16_AT_SKINNY = ["bf16_skinny_lds_n128_at_w4_s4", "bf16_skinny_lds_n128_at_w4_s4_whole_k"]


@pytest.mark.parametrize("M", [8, 16])
@pytest.mark.parametrize("NK", [(8192, 4096), (1000, 3008), (1000, 777)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_bf16_skinny_a_transposed_exact(gpu_available, M, NK):
    """bf16, M of 8 or 16, A stored K x M with its rows padded to 16 elements
    by NaN (which must never reach C): both streaming kernels forced, and the
    library's choice with and without a workspace, bit-exact on integer data
    with bias and ReLU.  K = 777 ends in a partial 32-row block of A, whose
    rows past K must read as zero."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=780 + M, dtype="bf16f32")
    As = A.t().contiguous()
    bias = make_bias(N, seed=781, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu", "T", "N")
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_BF16F32)
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    pad = (16 - M, 0, 0)
    runs = [(n, ids[n], ws) for n in BF16_AT_SKINNY] + [("auto", 0, None), ("auto ws", 0, ws)]
    for name, kid, w in runs:
        say(f"[bf16 A^T skinny] {name} M={M} N={N} K={K} lda=16 seed={780 + M}")
        C, _, _ = run_gemm(As, B, C0, 2.0, -1.0, kernel=kid, ws=w, bias=bias, activation="relu", op_a="T", pad=pad)
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)
    st, pl = tg.gemm_plan_query_general(tg.GEMM_DTYPE_BF16F32, 1, 0, M, N, K, 1.0, 0x1000, 16, 0x1000, N, 0.0,
                                        0x1000, N, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] in BF16_AT_SKINNY


BF16_AT1_SKINNY = ["bf16_skinny_lds_n128_at1_w4_s4", "bf16_skinny_lds_n128_at1_w4_s4_whole_k"]


@pytest.mark.parametrize("M", [1, 5, 12, 13])
@pytest.mark.parametrize("NK", [(8192, 4096), (1000, 777), (1008, 3008)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_bf16_skinny_a_transposed_any_m_exact(gpu_available, M, NK):
    """bf16 with A stored K x M whose rows are not whole 16-byte chunks (M of
    1, 5, 12 or 13; rows padded by 3 NaN elements, and A one element off
    4-byte alignment): both forms of the kernel that loads A 2 bytes a lane,
    forced, and the library's choice with and without a workspace, bit-exact
    on integer data with bias and ReLU.  Columns past M (the NaN padding and
    the next row) must never reach C; rows past K must read as zero."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=790 + M, dtype="bf16f32")
    As = A.t().contiguous()
    bias = make_bias(N, seed=791, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu", "T", "N")
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_BF16F32)
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    runs = [(n, ids[n], ws) for n in BF16_AT1_SKINNY] + [("auto", 0, None), ("auto ws", 0, ws)]
    for name, kid, w in runs:
        say(f"[bf16 A^T skinny, 2-byte A] {name} M={M} N={N} K={K} lda={M + 3} offset=1 seed={790 + M}")
        C, _, _ = run_gemm(As, B, C0, 2.0, -1.0, kernel=kid, ws=w, bias=bias, activation="relu", op_a="T",
                           pad=(3, 0, 0), offset=(1, 0, 0))
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)
    st, pl = tg.gemm_plan_query_general(tg.GEMM_DTYPE_BF16F32, 1, 0, M, N, K, 1.0, 0x1002, M + 3, 0x1000, N, 0.0,
                                        0x1000, N, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] in BF16_AT1_SKINNY


def test_bf16_skinny_a_transposed_any_m_random(gpu_available):
    """12 x 8192 x 8192, A stored K x 12, N(0,1) data, with and without a
    workspace: within the bf16 bound, and the same bits as the untransposed
    call (the same matrix-instruction inputs in the same order)."""
    M, N, K = 12, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=792, dist="normal", dtype="bf16f32")
    As = A.t().contiguous()
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_BF16F32)
    a, b = host_view(As), host_view(B)
    for w in (ws, None):
        say(f"[bf16 A^T skinny, 2-byte A] auto M={M} N={N} K={K} normal seed=792 ws={w is not None}")
        C, _, _ = run_gemm(As, B, C0, 1.0, 0.5, ws=w, op_a="T")
        r = oracle.error_ratio(C, oracle.gemm_ref(a, b, 1.0, 0.5, C0.numpy(), "T", "N"),
                               oracle.gemm_absbound(a, b, 1.0, 0.5, C0.numpy(), "T", "N"))
        say(f"[bf16 A^T skinny, 2-byte A] ratio {r:.3e}")
        assert r <= TOL["bf16f32"]
        C2, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=w)
        np.testing.assert_array_equal(C, C2)


@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_single_row_a_stored_transposed(gpu_available, dtype, op_b):
    """M = 1, A stored K x 1 (lda = 1): the untransposed layout's kernels,
    exact on integer data against the oracle's transposed product."""
    M, N, K = 1, 4096, 3008
    A, B, C0 = make_integer_inputs(M, N, K, seed=793, dtype=dtype)
    As, Bs = stored(A, B, "T", op_b)
    say(f"[single row A^T] {dtype} op_b={op_b} M={M} N={N} K={K} seed=793")
    C, _, _ = run_gemm(As, Bs, C0, 2.0, -1.0, op_a="T", op_b=op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref_of(As, Bs, C0, 2.0, -1.0, "T", op_b))


def test_bf16_skinny_a_transposed_random_full_size(gpu_available):
    """16 x 8192 x 8192, A stored K x M, N(0,1) data with a workspace: the
    bf16 error ratio, and the same bits as the untransposed call (the same
    matrix-instruction inputs in the same order)."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=4, dist="normal", dtype="bf16f32")
    As = A.t().contiguous()
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_BF16F32)
    say(f"[bf16 A^T skinny] auto M={M} N={N} K={K} normal seed=4 ws=True")
    C, _, _ = run_gemm(As, B, C0, 1.0, 0.5, ws=ws, op_a="T")
    a, b = host_view(As), host_view(B)
    r = oracle.error_ratio(C, oracle.gemm_ref(a, b, 1.0, 0.5, C0.numpy(), "T", "N"),
                           oracle.gemm_absbound(a, b, 1.0, 0.5, C0.numpy(), "T", "N"))
    say(f"[bf16 A^T skinny] ratio {r:.3e}")
    assert r <= TOL["bf16f32"]
    C2, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=ws)
    np.testing.assert_array_equal(C, C2)
