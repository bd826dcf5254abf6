"""GPU parity of the output-quantising epilogue: results written as bf16 or
OCP E4M3 (saturating) instead of fp32 C.

Integer operands give exact fp32 results; scaled by a power of two they
stay exact, so every kernel's output must equal the oracle's quantisation
of the exact result bit for bit (fp8 results past 448 exercise the
saturation).  On N(0,1) data the output must lie between the quantisations
of the oracle result minus and plus the error allowance of the fp32 paths:
rounding is monotonic, so any fp32 value inside the allowance rounds into
that interval."""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, padded_device, say

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}
OUTS = {"bf16": (tg.GEMM_OUT_BF16, torch.bfloat16), "fp8": (tg.GEMM_OUT_FP8, torch.float8_e4m3fn)}
U32 = 2.0 ** -24


def out_buffer(M, N, kind, pad=0, offset=0):
    """Device output view (M x N, leading dimension N + pad, `offset`
    elements into its buffer) filled with a NaN pattern."""
    _, tdt = OUTS[kind]
    ld = N + pad
    if kind == "fp8":
        buf = torch.full((M * ld + offset + 1,), 0x7F, dtype=torch.uint8, device="cuda")
        return buf[offset:offset + M * ld].view(M, ld)[:, :N].view(torch.float8_e4m3fn)
    buf = torch.full((M * ld + offset + 1,), float("nan"), dtype=tdt, device="cuda")
    return buf[offset:offset + M * ld].view(M, ld)[:, :N]


def dev(t):
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    return t.cuda()


def stored(A, B, op_a, op_b):
    return (A.t().contiguous() if op_a == "T" else A), (B.t().contiguous() if op_b == "T" else B)


def run_quant(A, B, C0, alpha, beta, kind, scale, kernel=0, ws=None, bias=None, act=None, op_a="N", op_b="N",
              pad=0, offset=0):
    M, N = C0.shape
    out = out_buffer(M, N, kind, pad, offset)
    Cd = C0.cuda() if beta != 0.0 else None
    tg.gemm(dev(A), dev(B), Cd, alpha=alpha, beta=beta, kernel=kernel, ws=ws,
            bias=bias.cuda() if bias is not None else None, activation=act, op_a=op_a, op_b=op_b, out=out,
            out_scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def quant_kernels(dtype, kind, op_a="N", op_b="N"):
    bit = 2 * (op_a == "T") + (op_b == "T")
    ot = OUTS[kind][0]
    return [k for k in tg.kernels() if k["dtype"] == DT[dtype] and (k["layouts"] >> bit) & 1
            and (k["outputs"] >> ot) & 1]


def runnable(dtype, kind, op_a, op_b, M, N, K, kid, ws_bytes):
    lda = K if op_a == "N" else M
    ldb = N if op_b == "N" else K
    epi = (0, 0, OUTS[kind][0], 0x2000, N, 0.0)
    st, pl = tg.gemm_plan_query_epi(DT[dtype], 0 if op_a == "N" else 1, 0 if op_b == "N" else 1, M, N, K, 1.0,
                                    0x1000, lda, 0x1000, ldb, 0.5, 0x1000, N, kid, epi, ws_bytes)
    return st == tg.GEMM_OK


LAYOUTS = {"f32": [("N", "N"), ("N", "T"), ("T", "N")], "bf16f32": [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")],
           "fp8f32": [("N", "T"), ("N", "N"), ("T", "N"), ("T", "T")]}


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16f32", "fp8f32"])
def test_every_quantising_kernel_exact(gpu_available, dtype, kind):
    """Integer data, beta != 0, bias and ReLU, scale 1/4: every kernel that
    writes the output type, in every layout it runs, bit-exact."""
    ran = 0
    for op_a, op_b in LAYOUTS[dtype]:
        for k in quant_kernels(dtype, kind, op_a, op_b):
            skinny = k["path"] in (tg.GEMM_PATH_SKINNY, tg.GEMM_PATH_SKINNY_SPLITK)
            M, N, K = (13, 1000, 3008) if skinny else (300, 264, 1024)
            ws = tg.workspace(M, N, K, dtype=DT[dtype])
            wsb = ws.numel() if ws is not None else 0
            if not runnable(dtype, kind, op_a, op_b, M, N, K, k["id"], wsb):
                continue
            A, B, C0 = make_integer_inputs(M, N, K, seed=1200 + k["id"], dtype=dtype)
            As, Bs = stored(A, B, op_a, op_b)
            bias = make_bias(N, seed=1201, integer=True)
            say(f"[quant exact] {dtype} -> {kind} {k['name']} op_a={op_a} op_b={op_b} M={M} N={N} K={K} "
                f"seed={1200 + k['id']}")
            got = run_quant(As, Bs, C0, 2.0, -1.0, kind, 0.25, kernel=k["id"], ws=ws, bias=bias, act="relu",
                            op_a=op_a, op_b=op_b)
            z = oracle.gemm_epilogue_ref(host_view(As), host_view(Bs), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu",
                                         op_a, op_b)
            np.testing.assert_array_equal(got, oracle.quantize(z, kind, 0.25), err_msg=k["name"])
            ran += 1
    assert ran >= 2


def allowance(A, B, C0, alpha, beta, dtype, op_a="N", op_b="N"):
    a, b = host_view(A), host_view(B)
    D = oracle.gemm_absbound(a, b, alpha, beta, C0.numpy(), op_a, op_b)
    if dtype == "fp8f32":
        return 7 * 2.0 ** -13 * oracle.gemm_groupmax(a, b, alpha, op_a, op_b) + (2e-6 + U32) * D
    return (TOL[dtype] + U32) * D


def check_interval(got, z, allow, kind, scale):
    lo = oracle.quantize(z - allow, kind, scale) if scale > 0 else oracle.quantize(z + allow, kind, scale)
    hi = oracle.quantize(z + allow, kind, scale) if scale > 0 else oracle.quantize(z - allow, kind, scale)
    # the scale product is itself rounded to fp32 (relative 2^-24)
    lo = np.minimum(lo, oracle.quantize((z - allow) * (1 - U32), kind, scale))
    hi = np.maximum(hi, oracle.quantize((z + allow) * (1 + U32), kind, scale))
    bad = (got < lo) | (got > hi)
    assert not np.any(bad), f"{int(bad.sum())} outputs outside the rounding interval"


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
@pytest.mark.parametrize("case", ["f32_4096", "bf16_nt_skinny", "fp8_nt", "f32_ksplit", "bf16_skinny"])
def test_quantised_random_paths(gpu_available, kind, case):
    """N(0,1) data through the library's own choice on the main paths (the
    fp32 ring, the bf16 N x K skinny, the fp8 ring, a tiled K split, the bf16
    decode split) with beta != 0 and a non-power-of-two scale."""
    dtype, M, N, K, op_b, with_ws = {
        "f32_4096": ("f32", 1024, 1024, 4096, "N", False),
        "bf16_nt_skinny": ("bf16f32", 16, 8192, 4096, "T", False),
        "fp8_nt": ("fp8f32", 512, 768, 2048, "T", False),
        "f32_ksplit": ("f32", 256, 512, 6000, "N", True),
        "bf16_skinny": ("bf16f32", 16, 4096, 8192, "N", True),
    }[case]
    A, B, C0 = make_random_inputs(M, N, K, seed=1210, dist="normal", dtype=dtype)
    As, Bs = stored(A, B, "N", op_b)
    ws = tg.workspace(M, N, K, dtype=DT[dtype]) if with_ws else None
    scale = 0.7
    say(f"[quant random] {case} -> {kind} M={M} N={N} K={K} seed=1210")
    got = run_quant(As, Bs, C0, 0.5, 0.25, kind, scale, ws=ws, op_b=op_b)
    z = oracle.gemm_ref(host_view(As), host_view(Bs), 0.5, 0.25, C0.numpy(), "N", op_b)
    check_interval(got, z, allowance(As, Bs, C0, 0.5, 0.25, dtype, "N", op_b), kind, scale)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_quantised_wave_tail_scale_path_and_layout(gpu_available, kind):
    """The last-wave split (top rows direct, bottom rows through the reduce),
    the K == 0 scale path (act(beta*C0 + bias)), and a padded, unaligned
    output (element stores)."""
    # 4352 x 4096 bf16 with a workspace: 17 x 16 tiles of 256 = one wave + 16
    M, N, K = 4352, 4096, 2048
    A, B, C0 = make_integer_inputs(M, N, K, seed=1220, dtype="bf16f32")
    ws = tg.workspace(M, N, K, dtype=tg.GEMM_DTYPE_BF16F32)
    st, pl = tg.gemm_plan_query_epi(tg.GEMM_DTYPE_BF16F32, 0, 0, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.0, 0, N, 0,
                                    (0, 0, OUTS[kind][0], 0x2000, N, 0.0), ws.numel())
    assert st == tg.GEMM_OK and pl["split_row"] > 0, pl
    say(f"[quant tail] {kind} M={M} N={N} K={K} split_row={pl['split_row']}")
    got = run_quant(A, B, C0, 1.0, 0.0, kind, 0.125, ws=ws)
    z = oracle.gemm_ref(host_view(A), host_view(B), 1.0, 0.0, C0.numpy())
    np.testing.assert_array_equal(got, oracle.quantize(z, kind, 0.125))
    # K == 0
    M, N = 37, 70
    C0 = torch.from_numpy(np.random.default_rng(1221).integers(-300, 300, size=(M, N)).astype(np.float32))
    bias = make_bias(N, seed=1222, integer=True)
    A0 = torch.zeros((M, 0), dtype=torch.float32)
    B0 = torch.zeros((0, N), dtype=torch.float32)
    say(f"[quant scale path] {kind} M={M} N={N} K=0")
    got = run_quant(A0, B0, C0, 1.0, 2.0, kind, 1.0, bias=bias, act="relu")
    np.testing.assert_array_equal(got, oracle.quantize(oracle.epilogue_ref(2.0 * C0.numpy().astype(np.float64),
                                                                              bias.numpy(), "relu"), kind))
    # padded and unaligned output through the fp32 ring
    M, N, K = 300, 264, 512
    A, B, C0 = make_integer_inputs(M, N, K, seed=1223, dtype="f32")
    say(f"[quant unaligned out] {kind} M={M} N={N} K={K} pad=3 offset=1")
    got = run_quant(A, B, C0, 1.0, 0.0, kind, 0.5, pad=3, offset=1)
    np.testing.assert_array_equal(got, oracle.quantize(oracle.gemm_ref(host_view(A), host_view(B), 1.0), kind, 0.5))


def test_quantised_saturation_and_nan(gpu_available):
    """Huge results saturate to +-448 in fp8 and overflow to infinity in
    bf16; a NaN in A gives NaN outputs in its row."""
    M, N, K = 64, 64, 64
    A, B, C0 = make_integer_inputs(M, N, K, seed=1230, dtype="f32")
    A[3, 5] = float("nan")
    for kind in ("bf16", "fp8"):
        say(f"[quant saturation] {kind}")
        got = run_quant(A, B, C0, 1e37, 0.0, kind, 100.0)
        z = oracle.gemm_ref(host_view(A), host_view(B), 1e37)
        expect = oracle.quantize(z, kind, 100.0)
        np.testing.assert_array_equal(np.isnan(got), np.isnan(expect))
        ok = ~np.isnan(expect)
        np.testing.assert_array_equal(got[ok], expect[ok])
        assert np.all(np.isnan(got[3]))
        if kind == "fp8":
            assert set(np.abs(got[ok & (z != 0)]).tolist()) == {448.0}
        else:
            assert np.all(np.isinf(got[ok & (z != 0)]))
