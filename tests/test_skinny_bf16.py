"""GPU parity of the bf16 skinny (M <= 16) split-K kernels: bf16 weights
streamed once, widened exactly to fp32, partials reduced in split order.

Integer operands make every sum exact, so results must equal the fp64
oracle bit for bit; random operands check the bf16 error bound.
Workspaces start full of NaN bit patterns."""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, ratio, run_gemm, say

pytestmark = pytest.mark.gpu

BF16 = tg.GEMM_DTYPE_BF16F32


def _skinny_ids():
    return {k["name"]: k["id"] for k in tg.kernels() if k["dtype"] == BF16 and k["layouts"] & 1
            and k["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK)}


def _ws(M, N, K):
    ws = tg.workspace(M, N, K, dtype=BF16)
    ws.fill_(0xFF)
    return ws


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("NK", [(8192, 8192), (4104, 8200), (1000, 3000)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_bf16_skinny_exact_every_variant(gpu_available, M, NK):
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=950 + M, dtype="bf16f32")
    bias = make_bias(N, seed=951, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(A), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu")
    ws = _ws(M, N, K)
    for name, kid in _skinny_ids().items():
        st, pl = tg.gemm_plan_query(BF16, M, N, K, 2.0, 0x1000, K, 0x1000, N, -1.0, 0x1000, N, kid, ws.numel())
        assert st == tg.GEMM_OK, name
        say(f"[bf16 skinny] {name} M={M} N={N} K={K} grid={pl['grid']} exact relu seed={950 + M}")
        C, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=kid, ws=ws, bias=bias, activation="relu")
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)


def test_bf16_skinny_random_and_deterministic(gpu_available):
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=960, dist="normal", dtype="bf16f32")
    ws = _ws(M, N, K)
    st, pl = tg.gemm_plan_query(BF16, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.5, 0x1000, N, 0, ws.numel())
    assert st == tg.GEMM_OK and pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK, pl
    say(f"[bf16 skinny] auto M={M} N={N} K={K} random seed=960")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=ws)
    r = ratio(C, A, B, C0, 1.0, 0.5)
    say(f"[bf16 skinny] ratio {r:.3e}")
    assert r <= TOL["bf16f32"]
    Ad, Bd = A.cuda(), B.cuda()
    outs = [tg.gemm(Ad, Bd, ws=ws) for _ in range(5)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_bf16_skinny_without_workspace(gpu_available):
    """16 x 8192 x 8192 without a workspace: the streaming kernel over the
    whole of K, within the bound and bit-identical to itself on repeats."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=961, dist="normal", dtype="bf16f32")
    st, pl = tg.gemm_plan_query(BF16, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.5, 0x1000, N, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] == "bf16_skinny_lds_n128_w4_s4_whole_k"
    say(f"[bf16 skinny] auto, no workspace M={M} N={N} K={K} random seed=961")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.5)
    r = ratio(C, A, B, C0, 1.0, 0.5)
    say(f"[bf16 skinny] ratio {r:.3e}")
    assert r <= TOL["bf16f32"]
    Ad, Bd = A.cuda(), B.cuda()
    outs = [tg.gemm(Ad, Bd) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_bf16_skinny_unaligned_a(gpu_available):
    """A one element off 16-byte alignment with a padded row: the library's
    choice (the tiled kernels) is still exact."""
    M, N, K = 9, 2048, 4096
    A, B, C0 = make_integer_inputs(M, N, K, seed=970, dtype="bf16f32")
    ws = _ws(M, N, K)
    say(f"[bf16 skinny] unaligned A M={M} N={N} K={K} offset=1 pad=3")
    C, Cd, _ = run_gemm(A, B, C0, 1.0, 1.0, ws=ws, pad=(3, 0, 0), offset=(1, 0, 0))
    np.testing.assert_array_equal(C.astype(np.float64),
                                  oracle.gemm_ref(host_view(A), host_view(B), 1.0, 1.0, C0.numpy()))
