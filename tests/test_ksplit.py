"""GPU parity of the tiled kernels' K split (partial products in a caller
workspace, reduced in split order).

Integer operands make every partial sum exact in fp32, so the split result
must equal the fp64 oracle bit for bit whatever the slice boundaries; random
operands check the error bound; repeated calls check determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, ratio, run_gemm, say

pytestmark = pytest.mark.gpu

F32, BF16 = tg.GEMM_DTYPE_F32, tg.GEMM_DTYPE_BF16F32


def _exact(A, B, C0, alpha, beta):
    return oracle.gemm_ref(host_view(A), host_view(B), alpha, beta, C0.numpy())


def _plan(dt, M, N, K, kernel, ws_bytes, alpha=1.0, beta=0.0):
    return tg.gemm_plan_query(dt, M, N, K, alpha, 0x1000, K, 0x1000, N, beta, 0x1000, N, kernel, ws_bytes)


def _nan_workspace(dt, M, N, K):
    ws = tg.workspace(M, N, K, dtype=dt)
    assert ws is not None
    ws.fill_(0xFF)             # NaN bit patterns: the contents on entry must not matter
    return ws


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_every_tiled_kernel_split_exact(gpu_available, dtype):
    """Each tiled kernel forced onto 256 x 512 x 6000 with a workspace: every
    tile size takes a 4-way split (slices of 1536, the last 1392)."""
    dt = F32 if dtype == "f32" else BF16
    M, N, K = 256, 512, 6000
    A, B, C0 = make_integer_inputs(M, N, K, seed=400, dtype=dtype)
    ref = _exact(A, B, C0, 2.0, 0.5)
    ws = _nan_workspace(dt, M, N, K)
    tiled = [k["id"] for k in tg.kernels()
             if k["dtype"] == dt and k["path"] == tg.GEMM_PATH_TILED and k["layouts"] & 1]
    ran = 0
    for kid in tiled:
        name = tg.gemm_kernel_query(kid)["name"]
        st, pl = _plan(dt, M, N, K, kid, ws.numel(), 2.0, 0.5)
        assert st == tg.GEMM_OK, name
        assert pl["splits"] == 4, (name, pl)
        say(f"[k-split exact] kernel={name} M={M} N={N} K={K} splits={pl['splits']} seed=400")
        C, _, _ = run_gemm(A, B, C0, 2.0, 0.5, kernel=kid, ws=ws)
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)
        ran += 1
    assert ran == len(tiled)


SHAPES = [
    # (M, N, K, expected tile, expected splits per dtype)
    (1024, 1024, 16384, {"f32": (256, 16), "bf16f32": (256, 16)}),
    (17, 8192, 8192, {"f32": (64, 2), "bf16f32": (128, 4)}),
    (100, 4096, 8192, {"f32": (128, 8), "bf16f32": (128, 8)}),
    (300, 704, 5000, {"f32": (64, 4), "bf16f32": (128, 4)}),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_auto_split_exact_and_random(gpu_available, dtype, shape):
    M, N, K, expect = shape
    dt = F32 if dtype == "f32" else BF16
    ws = _nan_workspace(dt, M, N, K)
    st, pl = _plan(dt, M, N, K, 0, ws.numel(), 1.0, -1.0)
    assert st == tg.GEMM_OK and (pl["tile_m"], pl["splits"]) == expect[dtype], pl
    A, B, C0 = make_integer_inputs(M, N, K, seed=401, dtype=dtype)
    say(f"[k-split auto] {dtype} M={M} N={N} K={K} tile={pl['tile_m']} splits={pl['splits']} exact seed=401")
    C, _, _ = run_gemm(A, B, C0, 1.0, -1.0, ws=ws)
    np.testing.assert_array_equal(C.astype(np.float64), _exact(A, B, C0, 1.0, -1.0))
    A, B, C0 = make_random_inputs(M, N, K, seed=402, dist="normal", dtype=dtype)
    say(f"[k-split auto] {dtype} M={M} N={N} K={K} random seed=402")
    C, _, _ = run_gemm(A, B, C0, 0.75, 0.25, ws=ws)
    r = ratio(C, A, B, C0, 0.75, 0.25)
    say(f"[k-split auto] ratio={r:.3e}")
    assert r <= TOL[dtype], r


def test_split_deterministic_and_matches_unsplit_bound(gpu_available):
    """Twenty calls give the same bits; the split and unsplit results both
    meet the bound (they differ only in summation order)."""
    M, N, K = 1024, 1024, 16384
    g = torch.Generator().manual_seed(403)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    B = torch.randn(K, N, generator=g).to(torch.bfloat16)
    Ad, Bd = A.cuda(), B.cuda()
    ws = tg.workspace(M, N, K, dtype=BF16)
    say(f"[k-split determinism] bf16 {M}x{N}x{K} x20")
    outs = [tg.gemm(Ad, Bd, ws=ws) for _ in range(20)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    C0 = torch.zeros(M, N)
    split = ratio(outs[0].cpu().numpy(), A, B, C0, 1.0, 0.0)
    plain = ratio(tg.gemm(Ad, Bd).cpu().numpy(), A, B, C0, 1.0, 0.0)
    say(f"[k-split determinism] ratio split={split:.3e} unsplit={plain:.3e}")
    assert split <= TOL["bf16f32"] and plain <= TOL["bf16f32"]
