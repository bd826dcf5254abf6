"""Operands of more than 2^31 bytes, and leading dimensions of 2^21
elements and more, on the GPU.

The kernels address operands through buffer resources with 32-bit offsets,
rebased per panel, slice or batch of k rows with 64-bit base arithmetic (the
size_t indexing of "Tiled matrix multiplication", "Code"), so such calls
keep their fast kernels: the streaming kernels for decode shapes with 2 GiB
of weights ("Avoid when": decode GEMV), the tiled kernels for a B with more
than 2^21 columns or an A whose rows lie 2^22 elements apart.  Inputs are
small integers, so every summation order gives the same exact result and the
GPU must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_integer_inputs

from gpu_helpers import host_view, oracle_ref, say

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32}


def _plan_name(dtype, M, N, K, lda, ldb, ws_bytes=0, op_a=0, op_b=0):
    st, pl = tg.gemm_plan_query_general(DT[dtype], op_a, op_b, M, N, K, 2.0, 0x1000, lda, 0x1000, ldb, -1.0,
                                        0x1000, N, 0, ws_bytes)
    assert st == tg.GEMM_OK
    return pl, tg.gemm_kernel_query(pl["kernel_id"])["name"]


def _exact(C, A, B, C0, alpha, beta):
    ref, _ = oracle_ref(A, B, C0, alpha, beta)
    np.testing.assert_array_equal(C.astype(np.float64), ref)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,N", [("f32", 65536), ("bf16f32", 131072)])
def test_decode_with_2gib_weights_streams(gpu_available, dtype, N):
    M, K = 16, 8192
    A, B, C0 = make_integer_inputs(M, N, K, seed=4100, dtype=dtype)
    assert B.numel() * B.element_size() >= 1 << 31
    Ad, Bd = A.cuda(), B.cuda()
    for with_ws in (False, True):
        ws = tg.workspace(M, N, K, dtype=DT[dtype]) if with_ws else None
        pl, name = _plan_name(dtype, M, N, K, K, N, ws.numel() if ws is not None else 0)
        assert pl["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK), name
        say(f"[large] {dtype} {M}x{N}x{K} B={B.numel() * B.element_size()} bytes workspace={with_ws} kernel={name}")
        Cd = C0.cuda()
        tg.gemm(Ad, Bd, Cd, alpha=2.0, beta=-1.0, ws=ws)
        _exact(Cd.cpu().numpy(), A, B, C0, 2.0, -1.0)
        del Cd, ws
    del Ad, Bd
    _free()


def test_tiled_b_with_more_than_2_21_columns(gpu_available):
    M, N, K = 64, (1 << 21) + 64, 256
    A, B, C0 = make_integer_inputs(M, N, K, seed=4200)
    assert B.numel() * 4 > 1 << 31
    pl, name = _plan_name("f32", M, N, K, K, N)
    assert "general" not in name and pl["path"] == tg.GEMM_PATH_TILED, name
    say(f"[large] f32 {M}x{N}x{K} ldb={N} kernel={name}")
    Ad, Bd, Cd = A.cuda(), B.cuda(), C0.cuda()
    tg.gemm(Ad, Bd, Cd, alpha=2.0, beta=-1.0)
    _exact(Cd.cpu().numpy(), A, B, C0, 2.0, -1.0)
    del Ad, Bd, Cd
    _free()


def test_tiled_a_with_rows_2_22_apart(gpu_available):
    """A's rows 2^22 + 2^18 floats apart inside a 9.1 GB buffer (its padding
    filled with NaN, which must never reach C): 256- and 128-row panels would
    span more than 2^31 bytes, 64-row ones do not."""
    M, N, K, lda = 512, 1024, 4096, (1 << 22) + (1 << 18)
    for tile in (128, 256):
        ring = [k["id"] for k in tg.kernels() if k["dtype"] == DT["f32"] and k["tile_m"] == tile
                and k["path"] == tg.GEMM_PATH_TILED and k["layouts"] & 1 and "general" not in k["name"]]
        assert ring
        for kid in ring:
            st, _ = tg.gemm_plan_query(DT["f32"], M, N, K, 2.0, 0x1000, lda, 0x1000, N, -1.0, 0x1000, N, kid, 0)
            assert st == tg.GEMM_ERR_UNSUPPORTED, (tile, kid)
    A, B, C0 = make_integer_inputs(M, N, K, seed=4300)
    pl, name = _plan_name("f32", M, N, K, lda, N)
    assert pl["tile_m"] == 64 and "general" not in name, name
    say(f"[large] f32 {M}x{N}x{K} lda={lda} kernel={name}")
    buf = torch.full((M * lda,), float("nan"), device="cuda")
    assert buf.numel() * 4 > 1 << 31
    Ad = buf.view(M, lda)[:, :K]
    Ad.copy_(A.cuda())
    Bd, Cd = B.cuda(), C0.cuda()
    tg.gemm(Ad, Bd, Cd, alpha=2.0, beta=-1.0)
    _exact(Cd.cpu().numpy(), A, B, C0, 2.0, -1.0)
    del buf, Ad, Bd, Cd
    _free()


@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("M,K", [(16, 777), (8, 1000), (16, 4096 + 40)])
def test_bf16_decode_a_stored_k_by_m_ragged_k(gpu_available, with_ws, M, K):
    """The bf16 streaming kernels with A stored K x M, K not a multiple of
    their 32-row blocks, A's stored rows padded to lda = M + 8 with NaN (the
    last block's rows past K must read as zero, and the padding only reaches
    rows of C that are never written)."""
    N = 2048
    A, B, C0 = make_integer_inputs(M, N, K, seed=4400 + K, dtype="bf16f32")
    lda = M + 8
    At = A.t().contiguous()                       # K x M
    buf = torch.full((K * lda,), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ad = buf.view(K, lda)[:, :M]
    Ad.copy_(At.cuda())
    ws = tg.workspace(M, N, K, dtype=DT["bf16f32"]) if with_ws else None
    pl, name = _plan_name("bf16f32", M, N, K, lda, N, ws.numel() if ws is not None else 0, op_a=1)
    assert "_at_" in name, name
    say(f"[bf16 AT ragged K] M={M} K={K} workspace={with_ws} kernel={name}")
    Cd = C0.cuda()
    tg.gemm(Ad, B.cuda(), Cd, alpha=2.0, beta=-1.0, op_a="T", ws=ws)
    _exact(Cd.cpu().numpy(), A, B, C0, 2.0, -1.0)
