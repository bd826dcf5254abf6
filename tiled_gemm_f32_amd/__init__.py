"""libgemm for MI355X (gfx950): C = alpha*(A x B) + beta*C on row-major operands.

The computation runs in hand-written HIP kernels inside ``libgemm.so``; this
package is a thin binding over its C ABI (``include/gemm.h``).  ``gemm_f32``,
``gemm_bf16f32`` and the other C entry points are re-exported with the same
names and arguments (integer device pointers and stream handles).
``gemm(A, B, C, alpha, beta)`` is a convenience over torch tensors that only
reads shapes, strides and pointers and forwards them.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401  (re-exported C ABI)
    EXPORTED, GEMM_ACT_GELU, GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_DTYPE_BF16F32, GEMM_DTYPE_F32, GEMM_DTYPE_FP8F32,
    GEMM_OP_N, GEMM_OP_T, GEMM_OUT_BF16, GEMM_OUT_F32, GEMM_OUT_FP8, Epilogue, gemm_bf16f32_epi, gemm_f32_epi,
    gemm_general, gemm_plan_query_general, gemm_plan_query_epi, GEMM_ERR_DEVICE, GEMM_ERR_INVALID_ARG,
    GEMM_ERR_LAUNCH, GEMM_ERR_UNSUPPORTED, GEMM_OK, GEMM_PATH_NONE, GEMM_PATH_SCALE,
    GEMM_PATH_SKINNY, GEMM_PATH_SKINNY_SPLITK, GEMM_PATH_TILED, GemmError, gemm_bf16f32,
    gemm_bf16f32_ex, gemm_bf16f32_ws, gemm_f32, gemm_f32_ex, gemm_f32_ws, gemm_kernel_count, gemm_kernel_query,
    gemm_plan_query, gemm_status_string, gemm_workspace_size, gemm_autotune, gemm_autotune_general, gemm_tuning_count,
    gemm_tuning_clear, gemm_tuning_save, gemm_tuning_load, load, gemm_general_noalloc, GEMM_ERR_SCRATCH,
    GEMM_STATIC_SCRATCH_BYTES)

__all__ = ["gemm", "gemm_f32", "gemm_bf16f32", "gemm_f32_ex", "gemm_bf16f32_ex", "gemm_f32_ws", "gemm_bf16f32_ws",
           "gemm_f32_epi", "gemm_bf16f32_epi", "Epilogue", "GEMM_ACT_NONE", "GEMM_ACT_RELU", "GEMM_ACT_GELU",
           "GEMM_OUT_F32", "GEMM_OUT_BF16", "GEMM_OUT_FP8", "gemm_plan_query_epi",
           "gemm_general", "gemm_plan_query_general", "GEMM_DTYPE_FP8F32", "GEMM_OP_N", "GEMM_OP_T",
           "gemm_workspace_size", "gemm_status_string", "gemm_kernel_count", "gemm_kernel_query",
           "gemm_plan_query", "GemmError", "kernels", "workspace", "autotune", "gemm_autotune",
           "gemm_autotune_general", "gemm_tuning_count",
           "gemm_tuning_clear", "gemm_tuning_save", "gemm_tuning_load", "gemm_general_noalloc",
           "GEMM_ERR_SCRATCH", "GEMM_STATIC_SCRATCH_BYTES"]


def _ld(t, what: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    rows, cols = t.shape
    if t.numel() == 0:
        return max(cols, 1)
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} must be row-major (stride(1) == 1); got strides {t.stride()}")
    return t.stride(0) if rows > 1 else max(cols, 1)


def workspace(M: int, N: int, K: int, device=None, dtype: int = GEMM_DTYPE_F32):
    """An uninitialised uint8 device tensor large enough for the split-K
    workspace paths of this shape and operand type (or None when none applies)."""
    import torch
    n = gemm_workspace_size(dtype, M, N, K)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


_ACTIVATIONS = {None: GEMM_ACT_NONE, "none": GEMM_ACT_NONE, "relu": GEMM_ACT_RELU, "gelu": GEMM_ACT_GELU}


def _dtype_of(t):
    import torch
    if t.dtype == torch.float32:
        return GEMM_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GEMM_DTYPE_BF16F32
    if t.dtype == torch.float8_e4m3fn:
        return GEMM_DTYPE_FP8F32
    raise TypeError(f"operands must be float32, bfloat16 or float8_e4m3fn (got {t.dtype})")


def gemm(A, B, C=None, alpha: float = 1.0, beta: float = 0.0, kernel: int = 0, stream=None, ws=None,
         bias=None, activation=None, op_a: str = "N", op_b: str = "N", out=None, out_scale: float = 1.0):
    """C = act(alpha * (op(A) @ op(B)) + beta * C + bias) on the current stream; returns C.

    A and B are CUDA tensors of one dtype: float32 (fp32 path), bfloat16
    (bf16 operands, fp32 accumulate) or float8_e4m3fn (fp8 operands, fp32
    accumulate).  ``op_a="T"`` means A is passed transposed (K x M), and
    ``op_b="T"`` that B is passed transposed (N x K); otherwise A is M x K and
    B is K x N.  C is float32 (M x N), allocated when None (then beta must be
    0).  All tensors must be row-major with unit stride along columns; padded
    leading dimensions are fine.  ``kernel`` forces a kernel id (0 = library
    choice).  ``ws`` is an optional device workspace tensor (see
    ``workspace()``) for the split-K paths.  ``bias`` is an optional float32
    device tensor of N elements added to every row; ``activation`` is None,
    "relu", "gelu" or a GEMM_ACT_* value.  Both are applied inside the
    kernels' epilogue.  ``out`` (optional) is a bfloat16 or float8_e4m3fn
    device tensor (M x N) that receives ``round(out_scale * result)`` instead
    of C (nearest-even; fp8 saturates at +-448); C is then only read, as C0,
    when beta != 0, and ``out`` is returned.
    """
    import torch

    if A.dtype != B.dtype:
        raise TypeError(f"A and B must have one dtype (got {A.dtype}, {B.dtype})")
    dt = _dtype_of(A)
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    if op_a not in ("N", "T") or op_b not in ("N", "T"):
        raise ValueError("op_a and op_b are 'N' or 'T'")
    M, K = A.shape if op_a == "N" else (A.shape[1], A.shape[0])
    K2, N = B.shape if op_b == "N" else (B.shape[1], B.shape[0])
    if K2 != K:
        raise ValueError(f"inner dimensions differ: op_a={op_a} {tuple(A.shape)}, op_b={op_b} {tuple(B.shape)}")
    out_type = GEMM_OUT_F32
    if out is not None:
        kinds = {torch.bfloat16: GEMM_OUT_BF16, torch.float8_e4m3fn: GEMM_OUT_FP8}
        if out.dtype not in kinds or tuple(out.shape) != (M, N) or not out.is_cuda:
            raise ValueError(f"out must be a bfloat16 or float8_e4m3fn device tensor of shape {(M, N)}")
        out_type = kinds[out.dtype]
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an input C")
        if out is None:
            C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if C is not None and (C.dtype != torch.float32 or tuple(C.shape) != (M, N) or not C.is_cuda):
        raise ValueError(f"C must be a float32 device tensor of shape {(M, N)}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    ldc = _ld(C, "C") if C is not None else max(N, 1)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    act = _ACTIVATIONS[activation] if activation is None or isinstance(activation, str) else int(activation)
    epi = None
    if bias is not None or act != GEMM_ACT_NONE or out is not None:
        if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda or bias.numel() != N
                                 or not bias.is_contiguous()):
            raise ValueError(f"bias must be a contiguous float32 device tensor of {N} elements")
        if out is not None:
            out_ptr = out.view(torch.uint8).data_ptr() if out_type == GEMM_OUT_FP8 else out.data_ptr()
            epi = Epilogue(bias.data_ptr() if bias is not None else None, act, out_type, out_ptr,
                           _ld(out, "out"), float(out_scale))
        else:
            epi = Epilogue(bias.data_ptr() if bias is not None else None, act)
    c_ptr = C.data_ptr() if C is not None else None
    args = (M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb, float(beta), c_ptr, ldc)
    ops = (GEMM_OP_N if op_a == "N" else GEMM_OP_T, GEMM_OP_N if op_b == "N" else GEMM_OP_T)
    with torch.cuda.device(A.device):
        wp, wb = (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (0, 0)
        if dt == GEMM_DTYPE_F32 and ops == (GEMM_OP_N, GEMM_OP_N):
            st = gemm_f32_ex(*args, kernel, epi, wp, wb, stream)
        elif dt == GEMM_DTYPE_BF16F32 and ops == (GEMM_OP_N, GEMM_OP_N):
            st = gemm_bf16f32_ex(*args, kernel, epi, wp, wb, stream)
        else:
            st = gemm_general(dt, ops[0], ops[1], *args, kernel, epi, wp, wb, stream)
    if st != GEMM_OK:
        raise GemmError(st, "gemm")
    return out if out is not None else C


def autotune(A, B, C, alpha: float = 1.0, beta: float = 0.0, ws=None, reps: int = 5, stream=None,
             op_a: str = "N", op_b: str = "N") -> dict:
    """Time every kernel that can run this call and record the fastest for
    calls of the same kind; returns the plan they now take.  C is scratch.
    Operands and ``op_a``/``op_b`` are as in ``gemm``."""
    import torch
    if op_a not in ("N", "T") or op_b not in ("N", "T"):
        raise ValueError("op_a and op_b are 'N' or 'T'")
    M, K = A.shape if op_a == "N" else (A.shape[1], A.shape[0])
    N = B.shape[1] if op_b == "N" else B.shape[0]
    dt = _dtype_of(A)
    wp, wb = (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (0, 0)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    ops = (GEMM_OP_N if op_a == "N" else GEMM_OP_T, GEMM_OP_N if op_b == "N" else GEMM_OP_T)
    with torch.cuda.device(A.device):
        st, pl = gemm_autotune_general(dt, *ops, M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"), B.data_ptr(),
                                       _ld(B, "B"), float(beta), C.data_ptr(), _ld(C, "C"), wp, wb, reps, stream)
    if st != GEMM_OK:
        raise GemmError(st, "autotune")
    return pl


def kernels() -> list:
    """Descriptions of every kernel in the library's table."""
    return [gemm_kernel_query(i) for i in range(1, gemm_kernel_count() + 1)]
