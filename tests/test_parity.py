"""GPU parity: the HIP kernels against the fp64 oracle.

Acceptance (per output entry, max over C):
    |C_gpu - C_ref| / (|alpha| * sum_k |A_ik||B_kj| + |beta||C0_ij|)
    <= 2e-6 for fp32 operands, <= 1e-5 for bf16 operands,
and exact equality where the denominator is 0.  Inputs are the seeded
synthetic workloads (tiled_gemm_f32_amd.workloads) at their full sizes, in
the launch configuration the library picks for them (the one the benchmark
times).  Every entry of C is checked for every workload, the bf16 8192 cube
included (its reference is computed in blocks of rows).
"""
import numpy as np
import pytest
import torch

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import WORKLOADS, make_inputs

from gpu_helpers import TOL, blocked_ratio, ratio, run_gemm, say

pytestmark = pytest.mark.gpu

FULL_CHECK = ["f32_256", "f32_4092_beta", "f32_4096", "f32_1000x3000x777", "f32_16x8192x8192"]


@pytest.mark.parametrize("name", FULL_CHECK)
def test_workload_full_matrix(gpu_available, name):
    w = WORKLOADS[name]
    A, B, C0 = make_inputs(w)
    st, pl = tg.gemm_plan_query(0 if w.dtype == "f32" else 1, w.M, w.N, w.K, w.alpha, 0x1000, w.K, 0x1000,
                                w.N, w.beta, 0x1000, w.N)
    say(f"[parity] {name} M={w.M} N={w.N} K={w.K} alpha={w.alpha} beta={w.beta} seed={w.seed} "
        f"kernel={tg.gemm_kernel_query(pl['kernel_id'])['name']}")
    C, _, _ = run_gemm(A, B, C0, w.alpha, w.beta)
    r = ratio(C, A, B, C0, w.alpha, w.beta)
    say(f"[parity] {name} ratio={r:.3e} tol={TOL[w.dtype]:.0e}")
    assert r <= TOL[w.dtype], r


def test_skinny_workspace_path_full_matrix(gpu_available):
    """The 16 x 8192 x 8192 workload through the split-K workspace path (the
    configuration the benchmark times), every entry checked."""
    w = WORKLOADS["f32_16x8192x8192"]
    A, B, C0 = make_inputs(w)
    ws = tg.workspace(w.M, w.N, w.K)
    say(f"[parity] {w.name} via workspace ({ws.numel()} bytes)")
    C, _, _ = run_gemm(A, B, C0, w.alpha, w.beta, ws=ws)
    r = ratio(C, A, B, C0, w.alpha, w.beta)
    say(f"[parity] {w.name} split-k ratio={r:.3e}")
    assert r <= TOL["f32"], r


@pytest.mark.timeout(1200)   # about 2.2 TFLOP of fp64 oracle work on the host cores
def test_bf16_8192_full_matrix(gpu_available):
    """The bf16 8192 cube in the benchmark's own launch (no workspace, the
    kernel the library picks), every one of the 67M entries of C compared
    with the oracle.  The host side works in blocks of rows so that the fp64
    reference and bound stay small."""
    w = WORKLOADS["bf16f32_8192"]
    A, B, C0 = make_inputs(w)
    st, pl = tg.gemm_plan_query(1, w.M, w.N, w.K, w.alpha, 0x1000, w.K, 0x1000, w.N, w.beta, 0x1000, w.N)
    say(f"[parity] {w.name} M=N=K={w.M} seed={w.seed} kernel={tg.gemm_kernel_query(pl['kernel_id'])['name']} "
        f"(every entry)")
    C, _, _ = run_gemm(A, B, C0, w.alpha, w.beta)
    assert np.isfinite(C).all()
    r = blocked_ratio(C, A, B, C0, w.alpha, w.beta, rows_per_block=1024)
    say(f"[parity] {w.name} ratio={r:.3e} tol={TOL['bf16f32']:.0e} over all {w.M * w.N} entries")
    assert r <= TOL["bf16f32"], r


def test_bf16_medium_full(gpu_available):
    """bf16 on a ragged 1000 x 1500 x 776 problem, every entry checked."""
    g = torch.Generator().manual_seed(41)
    A = torch.randn(1000, 776, generator=g).to(torch.bfloat16)
    B = torch.randn(776, 1500, generator=g).to(torch.bfloat16)
    C0 = torch.randn(1000, 1500, generator=g)
    say("[parity] bf16 1000x1500x776 alpha=1.5 beta=-0.5 seed=41")
    C, _, _ = run_gemm(A, B, C0, 1.5, -0.5)
    r = ratio(C, A, B, C0, 1.5, -0.5)
    assert r <= TOL["bf16f32"], r


def test_repeated_calls_are_bitwise_identical(gpu_available):
    """No atomics on any path: the same call gives the same bits every time."""
    for name in ["f32_1000x3000x777", "f32_16x8192x8192"]:
        w = WORKLOADS[name]
        A, B, C0 = make_inputs(w)
        say(f"[determinism] {name} x20")
        Ad, Bd = A.cuda(), B.cuda()
        first = None
        for _ in range(20):
            Cd = C0.cuda()
            tg.gemm(Ad, Bd, Cd, alpha=w.alpha, beta=w.beta)
            torch.cuda.synchronize()
            if first is None:
                first = Cd.clone()
            else:
                assert torch.equal(first, Cd)
    g = torch.Generator().manual_seed(5)
    A = torch.randn(1024, 1024, generator=g).to(torch.bfloat16).cuda()
    B = torch.randn(1024, 1024, generator=g).to(torch.bfloat16).cuda()
    say("[determinism] bf16 1024^3 x20")
    outs = [tg.gemm(A, B) for _ in range(20)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
