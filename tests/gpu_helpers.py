"""Helpers for the GPU parity tests: move seeded host inputs to the device,
call the library through its C ABI, bring C back, and compare with the
oracle.  Nothing here computes a GEMM."""
import sys

import numpy as np
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import bf16_bits, fp8_bytes

TOL = {"f32": 2e-6, "bf16f32": 1e-5}


def say(msg: str):
    """Name the case before its GPU step (flushed, so a crash still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def host_view(t: torch.Tensor):
    """numpy operand for the oracle: float32 array, uint16 bf16 bits or uint8 fp8 bytes."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    if t.dtype == torch.float8_e4m3fn:
        return fp8_bytes(t)
    return t.contiguous().numpy()


def padded_device(t: torch.Tensor, pad: int = 0, offset: int = 0, fill=float("nan")):
    """Device copy of t inside a wider buffer.

    The row stride becomes cols + pad (padding filled with ``fill``) and the
    view starts ``offset`` elements into the buffer (to exercise unaligned
    bases).  Returns (view, backing buffer).
    """
    if t.dtype == torch.float8_e4m3fn:
        # Bytes only (no fp8 arithmetic on the device); padding is the NaN code.
        view, buf = padded_device(t.view(torch.uint8), pad, offset, fill=0x7F)
        return view.view(torch.float8_e4m3fn), buf
    rows, cols = t.shape
    ld = cols + pad
    buf = torch.full((rows * ld + offset + 1,), fill, dtype=t.dtype, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(t.to("cuda"))
    return view, buf


def needs_workspace(kernel: int) -> bool:
    return kernel > 0 and tg.gemm_kernel_query(kernel)["path"] == tg.GEMM_PATH_SKINNY_SPLITK


def run_gemm(A, B, C0, alpha, beta, kernel=0, pad=(0, 0, 0), offset=(0, 0, 0), c_fill=None, ws=None,
             bias=None, activation=None, op_a="N", op_b="N"):
    """Run the library on host inputs; returns (C as float32 numpy, C device view, C buffer).

    A zero-filled workspace is allocated when a workspace kernel is forced
    and none is given.  bias (host float32, N values) and activation are
    passed to the fused epilogue."""
    Ad, _a = padded_device(A, pad[0], offset[0])
    Bd, _b = padded_device(B, pad[1], offset[1])
    if c_fill is None:
        Cd, cbuf = padded_device(C0, pad[2], offset[2])
    else:
        Cd, cbuf = padded_device(torch.full_like(C0, c_fill), pad[2], offset[2])
    if ws is None and needs_workspace(kernel):
        M, K = A.shape if op_a == "N" else A.shape[::-1]
        N = B.shape[1] if op_b == "N" else B.shape[0]
        dt = {torch.float32: tg.GEMM_DTYPE_F32, torch.bfloat16: tg.GEMM_DTYPE_BF16F32,
              torch.float8_e4m3fn: tg.GEMM_DTYPE_FP8F32}[A.dtype]
        ws = tg.workspace(M, N, K, dtype=dt)
    bd = bias.to("cuda") if bias is not None else None
    tg.gemm(Ad, Bd, Cd, alpha=alpha, beta=beta, kernel=kernel, ws=ws, bias=bd, activation=activation, op_a=op_a,
            op_b=op_b)
    torch.cuda.synchronize()
    return Cd.cpu().numpy(), Cd, cbuf


def oracle_ref(A, B, C0, alpha, beta):
    a, b = host_view(A), host_view(B)
    c0 = C0.numpy()
    return oracle.gemm_ref(a, b, alpha, beta, c0), oracle.gemm_absbound(a, b, alpha, beta, c0)


def ratio(C_gpu, A, B, C0, alpha, beta):
    ref, D = oracle_ref(A, B, C0, alpha, beta)
    return oracle.error_ratio(C_gpu, ref, D)


def blocked_ratio(C_gpu, A, B, C0, alpha, beta, rows_per_block=1024):
    """Error ratio over every entry of C, with the oracle run on blocks of
    rows (each block's fp64 reference and bound are all that is held)."""
    import time
    a, b, c0 = host_view(A), host_view(B), C0.numpy()
    worst = 0.0
    t0 = time.perf_counter()
    for i in range(0, a.shape[0], rows_per_block):
        j = min(i + rows_per_block, a.shape[0])
        ab, cb = np.ascontiguousarray(a[i:j]), np.ascontiguousarray(c0[i:j])
        ref = oracle.gemm_ref(ab, b, alpha, beta, cb)
        D = oracle.gemm_absbound(ab, b, alpha, beta, cb)
        worst = max(worst, oracle.error_ratio(C_gpu[i:j], ref, D))
        say(f"[oracle] rows {i}..{j - 1} of {a.shape[0]} checked ({time.perf_counter() - t0:.0f} s, "
            f"{oracle.num_threads()} threads)")
    return worst


def boundary_indices(n: int, tiles=(16, 32, 64, 128, 256), extra: int = 8, seed: int = 0):
    """Indices at tile boundaries (first/last of each tile) plus random ones."""
    idx = {0, n - 1}
    for t in tiles:
        for b in range(t, n, t):
            if b % 1024 in (0,) or b < 3 * t or b > n - 3 * t:
                idx.update({b - 1, b})
    rng = np.random.default_rng(seed)
    idx.update(rng.integers(0, n, size=extra).tolist())
    return sorted(i for i in idx if 0 <= i < n)
