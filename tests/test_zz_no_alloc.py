"""gemm_general_noalloc on the GPU: the library's static scratch stands in
for the caller's workspace, and the results equal those of gemm_general with
a workspace bit for bit (same kernels, same split, same reduction order) and
meet the oracle's bound.  Each case makes two calls in a row, the second on a
smaller problem, so the second runs over scratch that still holds the first
call's partial products."""
import numpy as np
import pytest
import torch

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_random_inputs

from gpu_helpers import TOL, ratio, say

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32}


def _args(dtype, op_b, M, N, K, seed):
    A, B, C0 = make_random_inputs(M, N, K, seed, dtype=dtype)
    Bs = B.t().contiguous() if op_b == tg.GEMM_OP_T else B
    ldb = K if op_b == tg.GEMM_OP_T else N
    return A, B, Bs, C0, ldb


def _split_used(dtype, op_b, M, N, K, ldb):
    st, pl = tg.gemm_plan_query_general(DT[dtype], tg.GEMM_OP_N, op_b, M, N, K, 1.0, 0x1000, K, 0x1000, ldb, 0.5,
                                        0x1000, N, 0, tg.GEMM_STATIC_SCRATCH_BYTES)
    assert st == tg.GEMM_OK
    return pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK or pl["splits"] > 1


CASES = [
    # (dtype, op_b, first (M, N, K), second, smaller (M, N, K))
    ("f32", tg.GEMM_OP_N, (16, 8192, 8192), (16, 2048, 4096)),
    ("bf16f32", tg.GEMM_OP_N, (16, 8192, 8192), (8, 1024, 4096)),
    ("bf16f32", tg.GEMM_OP_N, (512, 512, 8192), (256, 256, 4096)),
    ("f32", tg.GEMM_OP_N, (300, 520, 6144), (100, 130, 3072)),
    ("f32", tg.GEMM_OP_T, (16, 4096, 8192), (16, 1024, 2048)),
]


@pytest.mark.parametrize("dtype,op_b,first,second", CASES)
def test_noalloc_matches_workspace_call(gpu_available, dtype, op_b, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        A, B, Bs, C0, ldb = _args(dtype, op_b, M, N, K, seed=900 + i)
        assert _split_used(dtype, op_b, M, N, K, ldb), (M, N, K)
        say(f"[noalloc] {dtype} op_b={op_b} M={M} N={N} K={K} call {i + 1}")
        Ad, Bd = A.cuda(), Bs.cuda()
        C_ref, C_new = C0.cuda(), C0.cuda()
        need = tg.gemm_workspace_size(DT[dtype], M, N, K)
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        st = tg.gemm_general(DT[dtype], tg.GEMM_OP_N, op_b, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), ldb, 0.5,
                             C_ref.data_ptr(), N, 0, None, ws.data_ptr(), need, stream)
        assert st == tg.GEMM_OK
        st = tg.gemm_general_noalloc(DT[dtype], tg.GEMM_OP_N, op_b, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(),
                                     ldb, 0.5, C_new.data_ptr(), N, 0, None, stream)
        assert st == tg.GEMM_OK, tg.gemm_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(C_new, C_ref)
        r = ratio(C_new.cpu().numpy(), A, B, C0, 1.0, 0.5)
        say(f"[noalloc] ratio={r:.3e}")
        assert np.isfinite(r) and r <= TOL[dtype], r


def test_noalloc_rejects_beyond_scratch_on_device(gpu_available):
    """The size check comes before any launch: C stays untouched."""
    say("[noalloc] rejection 2048x2048x65536 bf16")
    C = torch.full((2048, 2048), 3.0, device="cuda")
    A = torch.zeros((2048, 65536), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((65536, 2048), dtype=torch.bfloat16, device="cuda")
    st = tg.gemm_general_noalloc(tg.GEMM_DTYPE_BF16F32, tg.GEMM_OP_N, tg.GEMM_OP_N, 2048, 2048, 65536, 1.0,
                                 A.data_ptr(), 65536, B.data_ptr(), 2048, 0.0, C.data_ptr(), 2048, 0, None,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == tg.GEMM_ERR_SCRATCH
    assert bool((C == 3.0).all())
