"""GPU parity of the last-wave split: a tile count just over a multiple of
the 256 compute units runs its top rows of tiles in whole waves, then the
leftover rows K-split over the idle compute units, reduced in split order.

Integer operands make every partial sum exact, so each case must equal the
fp64 oracle bit for bit whatever the slice boundaries; random operands check
the usual error bound.  Workspaces start full of NaN bit patterns.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, ratio, run_gemm, say

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}

CASES = [
    # (dtype, op_a, op_b, M, N, K, forced kernel: fp32 and fp8 choose 128 x 128 tiles here themselves)
    ("f32", "N", "N", 4352, 4096, 2048, "f32_mfma32_256x256x16_w2x2_a4b4_ring4"),
    ("bf16f32", "N", "N", 4352, 4096, 2048, ""),
    ("bf16f32", "N", "T", 4352, 4096, 2048, ""),
    ("fp8f32", "N", "T", 4352, 4096, 2048, "fp8_mfma32_256x256x128_w2x2_nt_lines"),
    ("f32", "T", "N", 4352, 4096, 2048, "f32_mfma32_256x256x16_w2x2_a4b4_tn_ring4"),
    ("f32", "T", "T", 4352, 4096, 2048, "f32_mfma32_256x256x16_w2x2_a4b4_tt_ring4"),
]
F32_RING256 = "f32_mfma32_256x256x16_w2x2_a4b4_ring4"


def kid(name):
    return next(k["id"] for k in tg.kernels() if k["name"] == name) if name else 0


def _stored(A, B, op_a, op_b):
    return (A.t().contiguous() if op_a == "T" else A), (B.t().contiguous() if op_b == "T" else B)


def _plan(dtype, op_a, op_b, M, N, K, ws_bytes, force=0):
    lda = K if op_a == "N" else M
    ldb = N if op_b == "N" else K
    return tg.gemm_plan_query_general(DT[dtype], 0 if op_a == "N" else 1, 0 if op_b == "N" else 1, M, N, K, 1.0,
                                      0x1000, lda, 0x1000, ldb, 0.5, 0x1000, N, force, ws_bytes)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}{c[2]}-{c[3]}x{c[4]}x{c[5]}")
def test_wave_tail_exact(gpu_available, case):
    dtype, op_a, op_b, M, N, K, force = case
    ws = tg.workspace(M, N, K, dtype=DT[dtype])
    ws.fill_(0xFF)
    st, pl = _plan(dtype, op_a, op_b, M, N, K, ws.numel(), kid(force))
    assert st == tg.GEMM_OK and pl["split_row"] > 0 and pl["splits"] >= 2, pl
    A, B, C0 = make_integer_inputs(M, N, K, seed=800, dtype=dtype)
    As, Bs = _stored(A, B, op_a, op_b)
    bias = make_bias(N, seed=801, integer=True)
    say(f"[wave tail] {dtype} op_a={op_a} op_b={op_b} M={M} N={N} K={K} split_row={pl['split_row']} "
        f"splits={pl['splits']} kernel={force or 'chosen'} exact, relu, seed=800")
    C, _, _ = run_gemm(As, Bs, C0, 1.0, -1.0, ws=ws, bias=bias, activation="relu", op_a=op_a, op_b=op_b,
                       kernel=kid(force))
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(Bs), 1.0, -1.0, C0.numpy(), bias.numpy(), "relu",
                                   op_a, op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_wave_tail_random(gpu_available, dtype):
    M, N, K = 4352, 4096, 2048
    ws = tg.workspace(M, N, K, dtype=DT[dtype])
    A, B, C0 = make_random_inputs(M, N, K, seed=802, dist="normal", dtype=dtype)
    force = kid(F32_RING256 if dtype == "f32" else "")
    assert _plan(dtype, "N", "N", M, N, K, ws.numel(), force)[1]["split_row"] > 0
    say(f"[wave tail] {dtype} random M={M} N={N} K={K} seed=802")
    C, _, _ = run_gemm(A, B, C0, 0.5, 0.25, ws=ws, kernel=force)
    rows = list(range(0, 64)) + list(range(4032, 4160)) + list(range(M - 64, M))   # both parts and the seam
    r = ratio(C[rows], A[rows], B, C0[rows], 0.5, 0.25)
    say(f"[wave tail] ratio {r:.3e}")
    assert r <= TOL[dtype]


def test_wave_tail_matches_plain_bound_and_is_deterministic(gpu_available):
    """Five calls give the same bits; the plain (workspace-free) call meets
    the same bound on the same sampled rows."""
    M, N, K = 4352, 4096, 4096
    g = torch.Generator().manual_seed(803)
    A = torch.randn(M, K, generator=g)
    B = torch.randn(K, N, generator=g)
    Ad, Bd = A.cuda(), B.cuda()
    ws = tg.workspace(M, N, K)
    force = kid(F32_RING256)
    assert _plan("f32", "N", "N", M, N, K, ws.numel(), force)[1]["split_row"] == 4096
    say(f"[wave tail] fp32 {M}x{N}x{K} x5 determinism")
    outs = [tg.gemm(Ad, Bd, ws=ws, kernel=force) for _ in range(5)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    rows = [0, 1, 4095, 4096, 4097, M - 1]
    C0 = torch.zeros(len(rows), N)
    tail = ratio(outs[0].cpu().numpy()[rows], A[rows], B, C0, 1.0, 0.0)
    plain = ratio(tg.gemm(Ad, Bd, kernel=force).cpu().numpy()[rows], A[rows], B, C0, 1.0, 0.0)
    say(f"[wave tail] ratio tail={tail:.3e} plain={plain:.3e}")
    assert tail <= TOL["f32"] and plain <= TOL["f32"]


LAST_WAVE = [
    # (dtype, op_a, op_b, M, N, K, with a workspace): 256^2 tiles would leave a mostly empty last wave,
    # so the choice is 128^2 tiles, unsplit.
    ("f32", "N", "N", 4352, 4096, 1040, True),
    ("f32", "N", "T", 3072, 6144, 528, False),
    ("bf16f32", "N", "N", 3072, 6144, 1040, False),
    ("bf16f32", "T", "N", 4352, 4096, 528, False),
    ("fp8f32", "N", "T", 4352, 4096, 1024, True),
    ("fp8f32", "T", "T", 4352, 4096, 2048, False),
    ("fp8f32", "N", "N", 4096, 4096, 1024, False),
]


@pytest.mark.parametrize("case", LAST_WAVE, ids=lambda c: f"{c[0]}-{c[1]}{c[2]}-{c[3]}x{c[4]}x{c[5]}-ws{int(c[6])}")
def test_last_wave_128_tiles_exact(gpu_available, case):
    """The calls that leave 256^2 tiles for 128^2 ones: exact on integer
    data, with beta and a bias, against the oracle."""
    dtype, op_a, op_b, M, N, K, with_ws = case
    ws = tg.workspace(M, N, K, dtype=DT[dtype]) if with_ws else None
    if ws is not None:
        ws.fill_(0xFF)
    st, pl = _plan(dtype, op_a, op_b, M, N, K, ws.numel() if ws is not None else 0)
    assert st == tg.GEMM_OK and pl["tile_m"] == 128 and pl["splits"] == 1 and pl["split_row"] == 0, pl
    A, B, C0 = make_integer_inputs(M, N, K, seed=804, dtype=dtype)
    As, Bs = _stored(A, B, op_a, op_b)
    bias = make_bias(N, seed=805, integer=True)
    say(f"[last wave] {dtype} op_a={op_a} op_b={op_b} M={M} N={N} K={K} ws={with_ws} kernel={pl['kernel_id']} "
        f"exact, seed=804")
    C, _, _ = run_gemm(As, Bs, C0, 1.0, -1.0, ws=ws, bias=bias, op_a=op_a, op_b=op_b)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(Bs), 1.0, -1.0, C0.numpy(), bias.numpy(), "none",
                                   op_a, op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref)
