"""Reference GEMM oracle -- TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU evaluation of ``C = alpha * (A x B) + beta * C0`` (the
definition that opens "GEMM Worklog I: Naive to Tiled" and that "A GEMM
Kernel, Step by Step" states as its one-call problem).  The arithmetic lives
in ``gemm_ref.c`` (plain C, OpenMP over rows); this module only builds it with
gcc and marshals numpy arrays.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it.

Arrays are 2-D numpy arrays whose last axis is contiguous; their row stride
(in elements) is passed as the leading dimension, so views into padded
buffers work unchanged.  fp32 operands are ``numpy.float32``; bf16 operands
are ``numpy.uint16`` bit patterns; fp8 operands (OCP E4M3) are
``numpy.uint8`` bytes.

Operand layouts: ``op_a="T"`` means the array passed as A holds A
transposed (K x M), ``op_b="T"`` that B holds B transposed (N x K).  The
oracle then multiplies the transposes, taken as plain copies.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_ref.c")
_LIB = os.path.join(_HERE, "libgemm_ref.so")

# -O2 without fast-math; contraction off so every operation is a plain IEEE op.
BUILD_FLAGS = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math"]


def build_cmd(out: str, src: str) -> list:
    """The gcc command that builds `src` into the shared library `out`."""
    return BUILD_FLAGS + ["-o", out, src, "-lm"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library; returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(build_cmd(tmp, _SRC), check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # The mutation tests point this at a deliberately broken build of the
    # same source to show that the pins catch it.
    path = os.environ.get("GEMM_ORACLE_LIB") or _LIB
    if path == _LIB and not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    sig = [i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, i64]
    for name in ("gemm_ref_f32in", "gemm_ref_bf16in", "gemm_ref_fp8in",
                 "gemm_absbound_f32in", "gemm_absbound_bf16in", "gemm_absbound_fp8in"):
        fn = getattr(lib, name)
        fn.argtypes = sig
        fn.restype = None
    lib.gemm_groupmax_fp8in.argtypes = [i64, i64, i64, dbl, vp, i64, vp, i64, vp, i64]
    lib.gemm_groupmax_fp8in.restype = None
    lib.epilogue_ref.argtypes = [i64, i64, vp, i64, vp, ctypes.c_int]
    lib.epilogue_ref.restype = None
    lib.quantize_ref.argtypes = [i64, i64, vp, i64, ctypes.c_int, dbl]
    lib.quantize_ref.restype = None
    lib.gemm_ref_num_threads.argtypes = []
    lib.gemm_ref_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ld(x: np.ndarray, what: str) -> int:
    if x.ndim != 2:
        raise ValueError(f"{what} must be 2-D")
    if x.size == 0:
        return max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != x.itemsize:
        raise ValueError(f"{what}: last axis must be contiguous")
    if x.strides[0] % x.itemsize:
        raise ValueError(f"{what}: row stride not a multiple of the element size")
    return max(x.strides[0] // x.itemsize, 1)


def _ptr(x: np.ndarray) -> int:
    return x.__array_interface__["data"][0]


_SUFFIX = {np.dtype(np.float32): "f32in", np.dtype(np.uint16): "bf16in", np.dtype(np.uint8): "fp8in"}


def _oriented(A, B, op_a, op_b):
    """A as M x K and B as K x N (copies of the transposes where asked)."""
    if op_a not in ("N", "T") or op_b not in ("N", "T"):
        raise ValueError("op_a and op_b are 'N' or 'T'")
    if op_a == "T":
        A = np.ascontiguousarray(A.T)
    if op_b == "T":
        B = np.ascontiguousarray(B.T)
    return A, B


def _run(kind: str, A, B, alpha, beta, C0, op_a="N", op_b="N"):
    if A.dtype != B.dtype or A.dtype not in _SUFFIX:
        raise TypeError("operands must both be float32, uint16 (bf16 bits) or uint8 (fp8 E4M3 bytes)")
    suffix = _SUFFIX[A.dtype]
    A, B = _oriented(A, B, op_a, op_b)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
    lda, ldb = _ld(A, "A"), _ld(B, "B")
    if C0 is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C0")
        c0p, ldc0 = None, max(N, 1)
    else:
        if C0.dtype != np.float32 or C0.shape != (M, N):
            raise ValueError("C0 must be float32 of shape (M, N)")
        c0p, ldc0 = _ptr(C0), _ld(C0, "C0")
    out = np.empty((M, N), dtype=np.float64)
    fn = getattr(_load(), f"gemm_{kind}_{suffix}")
    fn(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
       c0p, ldc0, _ptr(out), max(N, 1))
    return out


def gemm_ref(A, B, alpha=1.0, beta=0.0, C0=None, op_a="N", op_b="N") -> np.ndarray:
    """fp64 ``alpha * op(A) @ op(B) + beta * C0`` over the exact input values.

    The beta term is left out (C0 not read) when ``beta == 0``.
    """
    return _run("ref", A, B, alpha, beta, C0, op_a, op_b)


def gemm_absbound(A, B, alpha=1.0, beta=0.0, C0=None, op_a="N", op_b="N") -> np.ndarray:
    """fp64 ``|alpha| * |op(A)| @ |op(B)| + |beta| * |C0|`` -- the error-ratio denominator."""
    return _run("absbound", A, B, alpha, beta, C0, op_a, op_b)


def gemm_groupmax(A, B, alpha=1.0, op_a="N", op_b="N") -> np.ndarray:
    """fp8 operands only: ``|alpha| * sum over runs q of 8 consecutive k of
    max_k |op(A)[i][k] * op(B)[k][j]|`` (runs start at k = 0, the last may be
    short) -- the scale of the truncation a matrix unit that sums each run of
    8 products at a fixed precision below the run's largest can make."""
    if A.dtype != np.uint8 or B.dtype != np.uint8:
        raise TypeError("gemm_groupmax takes fp8 (uint8) operands")
    A, B = _oriented(A, B, op_a, op_b)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {A.shape} x {B.shape}")
    out = np.empty((M, N), dtype=np.float64)
    _load().gemm_groupmax_fp8in(M, N, K, float(alpha), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"),
                                _ptr(out), max(N, 1))
    return out


# The oracle's own names for the activations (see epilogue_ref in gemm_ref.c).
ACTIVATIONS = {"none": 0, "relu": 1, "gelu": 2}


def epilogue_ref(Z, bias=None, activation="none") -> np.ndarray:
    """fp64 ``act(Z + bias)`` with the bias broadcast along rows.

    ``Z`` is a finished GEMM result (any float array, M x N); ``bias`` is
    None or N float32 values; ``activation`` is "none", "relu" (max(z, 0),
    NaN kept) or "gelu" (z * Phi(z), erf form).  Returns a new array.
    """
    out = np.array(Z, dtype=np.float64, order="C", copy=True)
    if out.ndim != 2:
        raise ValueError("Z must be 2-D")
    M, N = out.shape
    bp = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError(f"bias must hold {N} values")
        bp = _ptr(bias)
    _load().epilogue_ref(M, N, _ptr(out), max(N, 1), bp, ACTIVATIONS[activation])
    return out


def gemm_epilogue_ref(A, B, alpha=1.0, beta=0.0, C0=None, bias=None, activation="none", op_a="N",
                      op_b="N") -> np.ndarray:
    """fp64 ``act(alpha * op(A) @ op(B) + beta * C0 + bias)``: gemm_ref, then epilogue_ref."""
    return epilogue_ref(gemm_ref(A, B, alpha, beta, C0, op_a, op_b), bias, activation)


# The oracle's own names for the output formats (see quantize_ref in gemm_ref.c).
OUTPUTS = {"bf16": 1, "fp8": 2}


def quantize(Z, kind, scale=1.0) -> np.ndarray:
    """fp64 values of ``Z * scale`` rounded to ``kind`` ("bf16", or "fp8" =
    OCP E4M3 saturating at +-448), nearest with ties to even.  Returns a new
    array of the same shape."""
    out = np.array(Z, dtype=np.float64, order="C", copy=True)
    flat = out.reshape(1, -1) if out.ndim != 2 else out
    M, N = flat.shape
    _load().quantize_ref(M, N, _ptr(flat), max(N, 1), OUTPUTS[kind], float(scale))
    return out


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().gemm_ref_num_threads())


def error_ratio(C_gpu: np.ndarray, C_ref: np.ndarray, D: np.ndarray) -> float:
    """``max |C_gpu - C_ref| / D``; where ``D == 0`` the two must be equal.

    Returns ``inf`` when any entry is NaN/Inf on one side only or differs
    where the denominator is zero.
    """
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    err = np.abs(C_gpu - C_ref)
    if not np.all(np.isfinite(err)):
        return float("inf")
    zero = D == 0
    if np.any(err[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(err[~zero] / D[~zero]))
