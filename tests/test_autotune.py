"""GPU: per-shape autotuning picks a kernel by timing, records it, and the
calls that follow take it and still match the oracle."""
import numpy as np
import pytest
import torch

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, padded_device, ratio, run_gemm, say
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture
def clean_table():
    tg.gemm_tuning_clear()
    yield
    tg.gemm_tuning_clear()


def _plan(dt, M, N, K, ws_bytes=0):
    return tg.gemm_plan_query(dt, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.0, 0x1000, N, 0, ws_bytes)[1]


def test_autotune_records_and_is_used(gpu_available, clean_table):
    M, N, K = 1000, 3000, 777
    A, B, C0 = make_random_inputs(M, N, K, seed=500, dist="uniform")
    Ad, Bd = A.cuda(), B.cuda()
    scratch = torch.empty(M, N, device="cuda")
    say(f"[autotune] f32 {M}x{N}x{K} reps=3")
    pl = tg.autotune(Ad, Bd, scratch, alpha=2.0, beta=-1.0, reps=3)
    assert tg.gemm_tuning_count() == 1
    name = tg.gemm_kernel_query(pl["kernel_id"])["name"]
    say(f"[autotune] chose {name} splits={pl['splits']}")
    assert _plan(tg.GEMM_DTYPE_F32, M, N, K)["kernel_id"] == pl["kernel_id"]
    C, _, _ = run_gemm(A, B, C0, 2.0, -1.0)
    r = ratio(C, A, B, C0, 2.0, -1.0)
    say(f"[autotune] ratio={r:.3e}")
    assert r <= TOL["f32"]


def test_autotune_with_workspace_exact(gpu_available, clean_table):
    """bf16 17 x 8192 x 8192 with a workspace: the candidates include every
    kernel with and without a K split; the recorded choice gives the exact
    integer result."""
    M, N, K = 17, 8192, 8192
    dt = tg.GEMM_DTYPE_BF16F32
    A, B, C0 = make_integer_inputs(M, N, K, seed=501, dtype="bf16f32")
    Ad, Bd = A.cuda(), B.cuda()
    ws = tg.workspace(M, N, K, dtype=dt)
    scratch = torch.empty(M, N, device="cuda")
    say(f"[autotune] bf16 {M}x{N}x{K} with workspace reps=3")
    pl = tg.autotune(Ad, Bd, scratch, alpha=1.0, beta=1.0, ws=ws, reps=3)
    name = tg.gemm_kernel_query(pl["kernel_id"])["name"]
    say(f"[autotune] chose {name} splits={pl['splits']}")
    assert _plan(dt, M, N, K, ws.numel())["kernel_id"] == pl["kernel_id"]
    C, _, _ = run_gemm(A, B, C0, 1.0, 1.0, ws=ws)
    ref = oracle.gemm_ref(host_view(A), host_view(B), 1.0, 1.0, C0.numpy())
    np.testing.assert_array_equal(C.astype(np.float64), ref)


@pytest.mark.parametrize("dtype,op_a,op_b", [("fp8f32", "N", "T"), ("bf16f32", "T", "N"), ("f32", "T", "T"),
                                             ("bf16f32", "N", "T")])
def test_autotune_transposed_layouts_exact(gpu_available, clean_table, dtype, op_a, op_b):
    """Tuning a transposed layout records a choice for that layout only; the
    tuned call equals the oracle bitwise on integer data."""
    M, N, K = 520, 1100, 512
    dt = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}[dtype]
    oa, ob = (tg.GEMM_OP_N if op_a == "N" else tg.GEMM_OP_T), (tg.GEMM_OP_N if op_b == "N" else tg.GEMM_OP_T)
    A, B, C0 = make_integer_inputs(M, N, K, seed=502, dtype=dtype)
    As = A.t().contiguous() if op_a == "T" else A
    Bs = B.t().contiguous() if op_b == "T" else B
    (Ad, _a), (Bd, _b) = padded_device(As), padded_device(Bs)
    scratch = torch.empty(M, N, device="cuda")

    def plan_of(a, b):
        return tg.gemm_plan_query_general(dt, a, b, M, N, K, 1.0, 0x1000, K if a == tg.GEMM_OP_N else M, 0x1000,
                                          N if b == tg.GEMM_OP_N else K, 0.0, 0x1000, N, 0, 0)[1]

    others = {(a, b): plan_of(a, b)["kernel_id"] for a in (0, 1) for b in (0, 1) if (a, b) != (oa, ob)}
    say(f"[autotune] {dtype} op_a={op_a} op_b={op_b} {M}x{N}x{K} reps=3 seed=502")
    pl = tg.autotune(Ad, Bd, scratch, alpha=2.0, beta=-1.0, reps=3, op_a=op_a, op_b=op_b)
    name = tg.gemm_kernel_query(pl["kernel_id"])["name"]
    say(f"[autotune] chose {name} splits={pl['splits']}")
    assert tg.gemm_tuning_count() == 1
    assert plan_of(oa, ob)["kernel_id"] == pl["kernel_id"]
    assert {k: plan_of(*k)["kernel_id"] for k in others} == others      # other layouts: untouched
    C, _, _ = run_gemm(As, Bs, C0, 2.0, -1.0, op_a=op_a, op_b=op_b)
    ref = oracle.gemm_ref(host_view(As), host_view(Bs), 2.0, -1.0, C0.numpy(), op_a, op_b)
    np.testing.assert_array_equal(C.astype(np.float64), ref)
