"""ctypes binding of libgemm's C ABI (include/gemm.h).

Every function here has the name and argument order of its C counterpart and
only converts arguments; all computation happens in libgemm.so.  Pointers are
plain integers (device addresses), streams are integer handles (0 = default
stream).  Loading fails loudly if the library has not been built: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_LAUNCH = 3
GEMM_ERR_DEVICE = 4
GEMM_ERR_SCRATCH = 5
# Bytes of the library's static device scratch (gemm_general_noalloc).
GEMM_STATIC_SCRATCH_BYTES = 32 << 20

GEMM_PATH_NONE = 0
GEMM_PATH_SCALE = 1
GEMM_PATH_TILED = 2
GEMM_PATH_SKINNY = 3
GEMM_PATH_SKINNY_SPLITK = 4

GEMM_DTYPE_F32 = 0
GEMM_DTYPE_BF16F32 = 1
GEMM_DTYPE_FP8F32 = 2

GEMM_OP_N = 0
GEMM_OP_T = 1

GEMM_ACT_NONE = 0
GEMM_ACT_RELU = 1
GEMM_ACT_GELU = 2
# gemm_output
GEMM_OUT_F32 = 0
GEMM_OUT_BF16 = 1
GEMM_OUT_FP8 = 2

# Every entry point include/gemm.h declares.
EXPORTED = ("gemm_f32", "gemm_bf16f32", "gemm_status_string", "gemm_kernel_count",
            "gemm_kernel_query", "gemm_plan_query", "gemm_f32_ex", "gemm_bf16f32_ex",
            "gemm_workspace_size", "gemm_f32_ws", "gemm_bf16f32_ws", "gemm_autotune", "gemm_tuning_count",
            "gemm_tuning_clear", "gemm_tuning_save", "gemm_tuning_load", "gemm_f32_epi", "gemm_bf16f32_epi",
            "gemm_general", "gemm_plan_query_general", "gemm_plan_query_epi", "gemm_autotune_general",
            "gemm_general_noalloc")


class KernelInfo(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("dtype", ctypes.c_int32), ("path", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("vec_a", ctypes.c_int32), ("vec_b", ctypes.c_int32),
                ("name", ctypes.c_char_p), ("layouts", ctypes.c_int32), ("outputs", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("kernel_id", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("threads", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("vec_a", ctypes.c_int32), ("vec_b", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("split_row", ctypes.c_int64)]


class Epilogue(ctypes.Structure):
    """gemm_epilogue: bias (device pointer to N floats, or 0), activation, and
    the output (type, device pointer, leading dimension, scale; type 0 = C)."""
    _fields_ = [("bias", ctypes.c_void_p), ("activation", ctypes.c_int32), ("out_type", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64), ("out_scale", ctypes.c_float)]


def _epi(epilogue):
    """None, an Epilogue, or a (bias_ptr, activation[, out_type, out_ptr, ldo, out_scale]) tuple -> ctypes
    argument."""
    if epilogue is None or isinstance(epilogue, Epilogue):
        return epilogue
    bias, act, *rest = epilogue
    out_type, out, ldo, scale = (list(rest) + [0, None, 0, 0.0][len(rest):])[:4]
    return Epilogue(bias or None, act, out_type, out or None, ldo, scale)


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gemm_status_string(status)} (status {status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libgemm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m tiled_gemm_f32_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    gemm_sig = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64]
    lib.gemm_f32.argtypes = gemm_sig + [vp]
    lib.gemm_bf16f32.argtypes = gemm_sig + [vp]
    epi = ctypes.POINTER(Epilogue)
    lib.gemm_f32_ex.argtypes = gemm_sig + [i32, epi, vp, i64, vp]
    lib.gemm_bf16f32_ex.argtypes = gemm_sig + [i32, epi, vp, i64, vp]
    lib.gemm_f32_epi.argtypes = gemm_sig + [epi, vp, i64, vp]
    lib.gemm_general.argtypes = [i32, i32, i32] + gemm_sig + [i32, epi, vp, i64, vp]
    lib.gemm_general.restype = ctypes.c_int
    lib.gemm_general_noalloc.argtypes = [i32, i32, i32] + gemm_sig + [i32, epi, vp]
    lib.gemm_general_noalloc.restype = ctypes.c_int
    lib.gemm_plan_query_general.argtypes = [i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32,
                                            i64, ctypes.POINTER(Plan)]
    lib.gemm_plan_query_general.restype = ctypes.c_int
    lib.gemm_plan_query_epi.argtypes = [i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32, epi,
                                        i64, ctypes.POINTER(Plan)]
    lib.gemm_plan_query_epi.restype = ctypes.c_int
    lib.gemm_bf16f32_epi.argtypes = gemm_sig + [epi, vp, i64, vp]
    lib.gemm_f32_ws.argtypes = gemm_sig + [vp, i64, vp]
    lib.gemm_bf16f32_ws.argtypes = gemm_sig + [vp, i64, vp]
    for fn in (lib.gemm_f32, lib.gemm_bf16f32, lib.gemm_f32_ex, lib.gemm_bf16f32_ex, lib.gemm_f32_ws,
               lib.gemm_bf16f32_ws, lib.gemm_f32_epi, lib.gemm_bf16f32_epi):
        fn.restype = ctypes.c_int
    lib.gemm_workspace_size.argtypes = [i32, i64, i64, i64]
    lib.gemm_workspace_size.restype = i64
    lib.gemm_status_string.argtypes = [ctypes.c_int]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_kernel_count.argtypes = []
    lib.gemm_kernel_count.restype = i32
    lib.gemm_kernel_query.argtypes = [i32, ctypes.POINTER(KernelInfo)]
    lib.gemm_kernel_query.restype = ctypes.c_int
    lib.gemm_plan_query.argtypes = [i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, i32, i64,
                                    ctypes.POINTER(Plan)]
    lib.gemm_plan_query.restype = ctypes.c_int
    lib.gemm_autotune.argtypes = [i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp, i64, i32, vp,
                                  ctypes.POINTER(Plan)]
    lib.gemm_autotune.restype = ctypes.c_int
    lib.gemm_autotune_general.argtypes = [i32, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp, i64,
                                          i32, vp, ctypes.POINTER(Plan)]
    lib.gemm_autotune_general.restype = ctypes.c_int
    lib.gemm_tuning_count.argtypes = []
    lib.gemm_tuning_count.restype = i32
    lib.gemm_tuning_clear.argtypes = []
    lib.gemm_tuning_clear.restype = None
    lib.gemm_tuning_save.argtypes = [ctypes.c_char_p]
    lib.gemm_tuning_save.restype = ctypes.c_int
    lib.gemm_tuning_load.argtypes = [ctypes.c_char_p]
    lib.gemm_tuning_load.restype = i32
    _lib = lib
    return lib


def gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_bf16f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, stream=0) -> int:
    return load().gemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, stream)


def gemm_f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel, epilogue=None, workspace=0,
                workspace_bytes=0, stream=0) -> int:
    return load().gemm_f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel, _epi(epilogue),
                              workspace, workspace_bytes, stream)


def gemm_f32_epi(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, epilogue, workspace=0, workspace_bytes=0,
                 stream=0) -> int:
    return load().gemm_f32_epi(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, _epi(epilogue), workspace,
                               workspace_bytes, stream)


def gemm_workspace_size(dtype, M, N, K) -> int:
    return int(load().gemm_workspace_size(dtype, M, N, K))


def gemm_bf16f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel, epilogue=None, workspace=0,
                    workspace_bytes=0, stream=0) -> int:
    return load().gemm_bf16f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel, _epi(epilogue),
                                  workspace, workspace_bytes, stream)


def gemm_bf16f32_epi(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, epilogue, workspace=0, workspace_bytes=0,
                     stream=0) -> int:
    return load().gemm_bf16f32_epi(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, _epi(epilogue), workspace,
                                   workspace_bytes, stream)


def gemm_bf16f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, stream=0) -> int:
    return load().gemm_bf16f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                                  stream)


def gemm_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel=0, epilogue=None,
                 workspace=0, workspace_bytes=0, stream=0) -> int:
    return load().gemm_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel,
                               _epi(epilogue), workspace, workspace_bytes, stream)


def gemm_general_noalloc(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel=0,
                         epilogue=None, stream=0) -> int:
    return load().gemm_general_noalloc(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                       force_kernel, _epi(epilogue), stream)


def gemm_plan_query_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel=0,
                            workspace_bytes=0):
    """(status, plan dict) for the choice gemm_general would make."""
    pl = Plan()
    st = load().gemm_plan_query_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                        force_kernel, workspace_bytes, ctypes.byref(pl))
    return st, {f: getattr(pl, f) for f, _ in Plan._fields_}


def gemm_plan_query_epi(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel=0,
                        epilogue=None, workspace_bytes=0):
    """(status, plan dict) for the choice gemm_general would make with this epilogue."""
    pl = Plan()
    st = load().gemm_plan_query_epi(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel,
                                    _epi(epilogue), workspace_bytes, ctypes.byref(pl))
    return st, {f: getattr(pl, f) for f, _ in Plan._fields_}


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(status).decode()


def gemm_kernel_count() -> int:
    return int(load().gemm_kernel_count())


def gemm_kernel_query(kid: int) -> dict:
    info = KernelInfo()
    st = load().gemm_kernel_query(kid, ctypes.byref(info))
    if st != GEMM_OK:
        raise GemmError(st, f"gemm_kernel_query({kid})")
    d = {f: getattr(info, f) for f, _ in KernelInfo._fields_}
    d["name"] = info.name.decode()
    return d


def gemm_plan_query(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel=0, workspace_bytes=0):
    """(status, plan dict) for the choice the library would make."""
    pl = Plan()
    st = load().gemm_plan_query(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel,
                                workspace_bytes, ctypes.byref(pl))
    return st, {f: getattr(pl, f) for f, _ in Plan._fields_}


def gemm_autotune(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace=0, workspace_bytes=0, reps=5,
                  stream=0):
    """(status, plan dict) after timing every candidate; C is scratch."""
    pl = Plan()
    st = load().gemm_autotune(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes, reps,
                              stream, ctypes.byref(pl))
    return st, {f: getattr(pl, f) for f, _ in Plan._fields_}


def gemm_autotune_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace=0,
                          workspace_bytes=0, reps=5, stream=0):
    """gemm_autotune for any operand type and layout (op_a, op_b as in gemm_general)."""
    pl = Plan()
    st = load().gemm_autotune_general(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                      workspace_bytes, reps, stream, ctypes.byref(pl))
    return st, {f: getattr(pl, f) for f, _ in Plan._fields_}


def gemm_tuning_count() -> int:
    return int(load().gemm_tuning_count())


def gemm_tuning_clear() -> None:
    load().gemm_tuning_clear()


def gemm_tuning_save(path: str) -> int:
    return load().gemm_tuning_save(path.encode())


def gemm_tuning_load(path: str) -> int:
    return int(load().gemm_tuning_load(path.encode()))
