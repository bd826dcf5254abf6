"""GPU parity of the fused epilogue, C = act(alpha*(A x B) + beta*C0 + bias)
("Tiled matrix multiplication", "Efficiency" and "Implementation notes":
bias and activation applied while the tile is still in registers).

The oracle is gemm_ref followed by epilogue_ref, in fp64.  Tolerance, per
element, with z the oracle's pre-activation value and D' the GEMM's
error-bound denominator plus |bias|:

* none, ReLU: |C - ref| <= (tol + 2^-24) * D'.  tol is the GEMM's own bound
  (fp32 2e-6, bf16 operands 1e-5); adding the bias in fp32 rounds once, at
  most 2^-24 * |z| <= 2^-24 * D'; ReLU is 1-Lipschitz, so it adds nothing.
* GELU: |C - ref| <= 1.13 * (tol + 2^-24) * D' + 6e-7 * |z|.  1.13 bounds
  the slope of x*Phi(x) (its maximum is Phi(sqrt 2) + sqrt 2 * phi(sqrt 2)
  = 1.1289); 6e-7 * |z| bounds the kernels' fp32 evaluation of
  z/2 * (1 + erf(z/sqrt 2)): the erf approximation they use (Abramowitz &
  Stegun 7.1.26) is within 1.5e-7, its fp32 evaluation adds at most about
  10 roundings of values below 1 (6e-7), halved by the z/2 factor, and the
  two final products add 2 * 2^-24 relative.

Where the bound is zero the two must be equal; NaN must match NaN.
Integer operands, integer bias and ReLU (or none) make every value exact,
so those cases compare bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, needs_workspace, run_gemm, say

pytestmark = pytest.mark.gpu

F32, BF16 = tg.GEMM_DTYPE_F32, tg.GEMM_DTYPE_BF16F32
U32 = 2.0 ** -24
GELU_SLOPE = 1.13
GELU_EVAL = 6e-7
ACTS = ["none", "relu", "gelu"]


def _did(dtype):
    return F32 if dtype == "f32" else BF16


def check_epilogue(C, A, B, C0, alpha, beta, bias, act, dtype):
    """Assert the per-element bound above; returns the worst err / allowance."""
    a, b = host_view(A), host_view(B)
    c0 = C0.numpy()
    bias_np = bias.numpy() if bias is not None else None
    z = oracle.gemm_epilogue_ref(a, b, alpha, beta, c0, bias_np, "none")
    ref = oracle.epilogue_ref(z, None, act)
    D = oracle.gemm_absbound(a, b, alpha, beta, c0)
    if bias_np is not None:
        D = D + np.abs(bias_np.astype(np.float64))
    t = TOL[dtype] + U32
    allow = GELU_SLOPE * t * D + GELU_EVAL * np.abs(z) if act == "gelu" else t * D
    C = np.asarray(C, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(C), nan_ref), "NaN positions differ"
    err = np.abs(C - ref)[~nan_ref]
    allow = allow[~nan_ref]
    assert np.all(np.isfinite(err)), "non-finite difference"
    bad = err > allow
    assert not np.any(bad), f"{int(bad.sum())} elements out of bound; worst excess {float(np.max(err - allow)):.3e}"
    nz = allow > 0
    return float(np.max(err[nz] / allow[nz])) if np.any(nz) else 0.0


def _exact_epilogue(A, B, C0, alpha, beta, bias, act):
    return oracle.gemm_epilogue_ref(host_view(A), host_view(B), alpha, beta, C0.numpy(),
                                    bias.numpy() if bias is not None else None, act)


def _kernels(did):
    """Kernels of this operand type that run untransposed operands."""
    return [k["id"] for k in tg.kernels() if k["dtype"] == did and k["layouts"] & 1]


def _skinny(kid):
    return tg.gemm_kernel_query(kid)["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK)


def _runnable(did, M, N, K, kid, beta=0.5):
    wsb = tg.gemm_workspace_size(did, M, N, K) if needs_workspace(kid) else 0
    st, _ = tg.gemm_plan_query(did, M, N, K, 1.0, 0x1000, K, 0x1000, N, beta, 0x1000, N, kid, wsb)
    return st == tg.GEMM_OK


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("act", ACTS)
def test_every_kernel_random(gpu_available, dtype, act):
    """Every kernel, forced, on a ragged multi-tile shape; the scale
    1/sqrt(K) keeps the pre-activation values near the bend of GELU."""
    did = _did(dtype)
    ran = 0
    for kid in _kernels(did):
        name = tg.gemm_kernel_query(kid)["name"]
        M = 16 if _skinny(kid) else 300
        N, K = 520, 1030
        if not _runnable(did, M, N, K, kid):
            continue
        A, B, C0 = make_random_inputs(M, N, K, seed=500 + kid, dist="normal", dtype=dtype)
        bias = make_bias(N, seed=600 + kid)
        alpha = 1.0 / np.sqrt(K)
        say(f"[epilogue random] kernel={name} act={act} M={M} N={N} K={K} seed={500 + kid}")
        C, _, _ = run_gemm(A, B, C0, alpha, 0.5, kernel=kid, bias=bias, activation=act)
        r = check_epilogue(C, A, B, C0, alpha, 0.5, bias, act, dtype)
        say(f"[epilogue random] worst err/allowance {r:.3e}")
        ran += 1
    assert ran >= 4


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_every_kernel_integer_exact(gpu_available, dtype):
    """Integer operands and bias: none and ReLU are exact, bit for bit."""
    did = _did(dtype)
    for kid in _kernels(did):
        name = tg.gemm_kernel_query(kid)["name"]
        M = 13 if _skinny(kid) else 270
        N, K = 264, 200
        if not _runnable(did, M, N, K, kid, beta=-1.0):
            continue
        A, B, C0 = make_integer_inputs(M, N, K, seed=510 + kid, dtype=dtype)
        bias = make_bias(N, seed=610 + kid, integer=True)
        for act in ("none", "relu"):
            say(f"[epilogue exact] kernel={name} act={act} M={M} N={N} K={K} seed={510 + kid}")
            C, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=kid, bias=bias, activation=act)
            np.testing.assert_array_equal(C.astype(np.float64), _exact_epilogue(A, B, C0, 2.0, -1.0, bias, act),
                                          err_msg=f"{name} {act}")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_unaligned_and_padded_c(gpu_available, dtype, act):
    """C one element off 16-byte alignment with a padded row stride: the
    kernels' element-wise store path, with the library's choice of kernel."""
    M, N, K = 300, 264, 136
    A, B, C0 = make_random_inputs(M, N, K, seed=520, dist="normal", dtype=dtype)
    bias = make_bias(N, seed=620)
    alpha = 1.0 / np.sqrt(K)
    say(f"[epilogue unaligned C] {dtype} act={act} M={M} N={N} K={K} c_offset=1 c_pad=3")
    C, _, _ = run_gemm(A, B, C0, alpha, -0.75, pad=(0, 0, 3), offset=(0, 0, 1), bias=bias, activation=act)
    check_epilogue(C, A, B, C0, alpha, -0.75, bias, act, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("act", ACTS)
def test_tiled_k_split(gpu_available, dtype, act):
    """A tiled K split applies the epilogue once, in its reduce step."""
    did = _did(dtype)
    M, N, K = 256, 512, 6000
    ws = tg.workspace(M, N, K, dtype=did)
    ws.fill_(0xFF)
    st, pl = tg.gemm_plan_query(did, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.5, 0x1000, N, 0, ws.numel())
    assert st == tg.GEMM_OK and pl["splits"] > 1, pl
    A, B, C0 = make_integer_inputs(M, N, K, seed=530, dtype=dtype)
    bias = make_bias(N, seed=630, integer=True)
    say(f"[epilogue k-split] {dtype} act={act} M={M} N={N} K={K} splits={pl['splits']} integer seed=530")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=ws, bias=bias, activation=act)
    if act == "gelu":
        check_epilogue(C, A, B, C0, 1.0, 0.5, bias, act, dtype)
    else:
        np.testing.assert_array_equal(C.astype(np.float64), _exact_epilogue(A, B, C0, 1.0, 0.5, bias, act))
    A, B, C0 = make_random_inputs(M, N, K, seed=531, dist="normal", dtype=dtype)
    bias = make_bias(N, seed=631)
    alpha = 1.0 / np.sqrt(K)
    say(f"[epilogue k-split] {dtype} act={act} random seed=531")
    C, _, _ = run_gemm(A, B, C0, alpha, 0.5, ws=ws, bias=bias, activation=act)
    check_epilogue(C, A, B, C0, alpha, 0.5, bias, act, dtype)


@pytest.mark.parametrize("act", ACTS)
def test_skinny_split(gpu_available, act):
    """fp32 M <= 16 with a workspace: the skinny split path's reduce kernel."""
    M, N, K = 7, 1000, 8192
    ws = tg.workspace(M, N, K)
    ws.fill_(0xFF)
    st, pl = tg.gemm_plan_query(F32, M, N, K, 1.0, 0x1000, K, 0x1000, N, 1.0, 0x1000, N, 0, ws.numel())
    assert st == tg.GEMM_OK and pl["path"] == tg.GEMM_PATH_SKINNY_SPLITK, pl
    A, B, C0 = make_random_inputs(M, N, K, seed=540, dist="normal")
    bias = make_bias(N, seed=640)
    alpha = 1.0 / np.sqrt(K)
    say(f"[epilogue skinny split] act={act} M={M} N={N} K={K} seed=540")
    C, _, _ = run_gemm(A, B, C0, alpha, 1.0, ws=ws, bias=bias, activation=act)
    check_epilogue(C, A, B, C0, alpha, 1.0, bias, act, "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("act", ACTS)
def test_scale_path(gpu_available, dtype, act):
    """K == 0 and alpha == 0 give act(beta*C0 + bias); with beta == 0, C is
    not read (NaN-filled) and the result is act(bias)."""
    did = _did(dtype)
    M, N = 70, 130
    bias = make_bias(N, seed=650)
    for K, alpha, beta in [(0, 1.0, 0.5), (40, 0.0, -2.0), (40, 0.0, 0.0)]:
        st, pl = tg.gemm_plan_query(did, M, N, K, alpha, 0x1000, max(K, 1), 0x1000, N, beta, 0x1000, N, 0, 0)
        assert st == tg.GEMM_OK and pl["path"] == tg.GEMM_PATH_SCALE, pl
        A, B, C0 = make_random_inputs(M, N, K, seed=550, dist="normal", dtype=dtype)
        say(f"[epilogue scale] {dtype} act={act} M={M} N={N} K={K} alpha={alpha} beta={beta}")
        fill = float("nan") if beta == 0.0 else None
        C, _, _ = run_gemm(A, B, C0, alpha, beta, c_fill=fill, bias=bias, activation=act)
        check_epilogue(C, A, B, C0, alpha, beta, bias, act, dtype)     # beta*C0 + bias rounds once in fp32
        if beta == 0.0 and act != "gelu":
            np.testing.assert_array_equal(C.astype(np.float64), _exact_epilogue(A, B, C0, alpha, beta, bias, act))


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
@pytest.mark.parametrize("M", [9, 300])
def test_relu_keeps_nan(gpu_available, dtype, M):
    """NaN in C0 (beta != 0) reaches exactly its own output through ReLU."""
    N, K = 264, 64
    A, B, C0 = make_integer_inputs(M, N, K, seed=560, dtype=dtype)
    rng = np.random.default_rng(560)
    C0[torch.as_tensor(rng.integers(0, M, 20)), torch.as_tensor(rng.integers(0, N, 20))] = float("nan")
    bias = make_bias(N, seed=660, integer=True)
    say(f"[epilogue relu NaN] {dtype} M={M} N={N} K={K}")
    C, _, _ = run_gemm(A, B, C0, 1.0, 1.0, bias=bias, activation="relu")
    ref = _exact_epilogue(A, B, C0, 1.0, 1.0, bias, "relu")
    np.testing.assert_array_equal(C.astype(np.float64), ref)     # NaN == NaN in assert_array_equal


def _abi_args(A, B, C, M, N, K, alpha, beta):
    return (M, N, K, alpha, A.data_ptr(), K, B.data_ptr(), N, beta, C.data_ptr(), N)


@pytest.mark.parametrize("dtype", ["f32", "bf16f32"])
def test_epi_entry_points(gpu_available, dtype):
    """gemm_f32_epi / gemm_bf16f32_epi through the C ABI: a NULL descriptor
    and an empty one (no bias, no activation) both give the plain call's
    bits; a GELU descriptor meets the bound."""
    M, N, K = 520, 776, 392
    A, B, C0 = make_random_inputs(M, N, K, seed=570, dist="normal", dtype=dtype)
    bias = make_bias(N, seed=670)
    Ad, Bd, biasd = A.cuda(), B.cuda(), bias.cuda()
    plain_fn = tg.gemm_f32 if dtype == "f32" else tg.gemm_bf16f32
    epi_fn = tg.gemm_f32_epi if dtype == "f32" else tg.gemm_bf16f32_epi
    alpha = 1.0 / np.sqrt(K)
    outs = []
    for desc in ("plain", None, tg.Epilogue(None, tg.GEMM_ACT_NONE)):
        Cd = C0.cuda()
        say(f"[epilogue C ABI] {dtype} {M}x{N}x{K} descriptor={desc if desc is None or desc == 'plain' else 'empty'}")
        if desc == "plain":
            st = plain_fn(*_abi_args(Ad, Bd, Cd, M, N, K, alpha, 0.5), 0)
        else:
            st = epi_fn(*_abi_args(Ad, Bd, Cd, M, N, K, alpha, 0.5), desc, 0, 0, 0)
        assert st == tg.GEMM_OK
        torch.cuda.synchronize()
        outs.append(Cd.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    Cd = C0.cuda()
    say(f"[epilogue C ABI] {dtype} {M}x{N}x{K} gelu with bias")
    st = epi_fn(*_abi_args(Ad, Bd, Cd, M, N, K, alpha, 0.5), tg.Epilogue(biasd.data_ptr(), tg.GEMM_ACT_GELU),
                0, 0, 0)
    assert st == tg.GEMM_OK
    torch.cuda.synchronize()
    check_epilogue(Cd.cpu().numpy(), A, B, C0, alpha, 0.5, bias, "gelu", dtype)


def test_bench_shapes_sampled(gpu_available):
    """The benchmark's fp32 4096^3 and bf16 8192^3 calls with bias and GELU,
    checked on sampled rows and columns."""
    from gpu_helpers import boundary_indices
    for dtype, n in (("f32", 4096), ("bf16f32", 8192)):
        A, B, C0 = make_random_inputs(n, n, n, seed=580, dist="normal", dtype=dtype)
        bias = make_bias(n, seed=680)
        alpha = 1.0 / np.sqrt(n)
        say(f"[epilogue bench shape] {dtype} {n}^3 gelu seed=580")
        Ad, Bd, Cd = A.cuda(), B.cuda(), C0.cuda()
        tg.gemm(Ad, Bd, Cd, alpha=alpha, beta=0.5, bias=bias.cuda(), activation="gelu")
        torch.cuda.synchronize()
        C = Cd.cpu().numpy()
        rng = np.random.default_rng(3)
        rows = sorted(set(boundary_indices(n, extra=0, seed=1)[::8]) | set(rng.integers(0, n, 8).tolist()))
        cols = sorted(set(boundary_indices(n, extra=0, seed=2)[::8]) | set(rng.integers(0, n, 8).tolist()))
        check_epilogue(C[rows], A[rows], B, C0[rows], alpha, 0.5, bias, "gelu", dtype)
        check_epilogue(C[:, cols], A, B[:, cols].contiguous(), C0[:, cols].contiguous(), alpha, 0.5,
                       bias[cols].contiguous(), "gelu", dtype)
