"""GPU parity of the skinny kernels for B stored N x K (M <= 16, the
decode-GEMV layout of a linear layer's weights): fp32, bf16 and fp8 (OCP
E4M3) operands, with and without a K split through the workspace.

Integer operands make every sum exact (for fp8 too: products of |v| <= 4
lie within 2^4 of each other, far inside the matrix unit's 2^-13 run
truncation), so results must equal the fp64 oracle bit for bit.  Random
operands meet the error ratio of the untransposed paths (2e-6 fp32, 1e-5
bf16) and, for fp8, the run-truncation bound of the fp8 kernels.
Workspaces start full of NaN bit patterns."""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import TOL, host_view, run_gemm, say
from test_layouts import check as layout_check

pytestmark = pytest.mark.gpu

DT = {"f32": tg.GEMM_DTYPE_F32, "bf16f32": tg.GEMM_DTYPE_BF16F32, "fp8f32": tg.GEMM_DTYPE_FP8F32}
ALL = ["f32", "bf16f32", "fp8f32"]
ESZ = {"f32": 4, "bf16f32": 2, "fp8f32": 1}
OP_N, OP_T = tg.GEMM_OP_N, tg.GEMM_OP_T


def nt_kernels(dtype):
    return {k["name"]: k for k in tg.kernels() if k["dtype"] == DT[dtype] and "skinny_nt" in k["name"]}


def nan_ws(M, N, K, dtype):
    """NaN-filled workspace of the advertised size (None when no path needs one)."""
    ws = tg.workspace(M, N, K, dtype=DT[dtype])
    if ws is not None:
        ws.fill_(0xFF)
    return ws


def nbytes(ws):
    return ws.numel() if ws is not None else 0


def to_dev(t):
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    return t.cuda()


def plan(dtype, M, N, K, kid=0, ws_bytes=0, lda=None, ldb=None):
    return tg.gemm_plan_query_general(DT[dtype], OP_N, OP_T, M, N, K, 1.0, 0x1000, lda or K, 0x1000, ldb or K, 0.5,
                                      0x1000, N, kid, ws_bytes)


def ref_nt(A, Bt, C0, alpha, beta, bias=None, act="none"):
    a, b = host_view(A), host_view(Bt)
    return oracle.gemm_epilogue_ref(a, b, alpha, beta, C0.numpy(), None if bias is None else bias.numpy(), act,
                                    "N", "T")


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("NK", [(8192, 4096), (1000, 3008), (40, 12288), (33, 64)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_skinny_nt_exact_every_variant(gpu_available, dtype, M, NK):
    """Every variant, forced, on integer data: bit-exact, with bias and ReLU."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=1100 + M, dtype=dtype)
    Bt = B.t().contiguous()
    bias = make_bias(N, seed=1101, integer=True)
    ref = ref_nt(A, Bt, C0, 2.0, -1.0, bias, "relu")
    ws = nan_ws(M, N, K, dtype)
    for name, k in nt_kernels(dtype).items():
        st, pl = plan(dtype, M, N, K, k["id"], nbytes(ws))
        assert st == tg.GEMM_OK, name
        say(f"[skinny nt] {name} M={M} N={N} K={K} grid={pl['grid']} exact relu seed={1100 + M}")
        C, _, _ = run_gemm(A, Bt, C0, 2.0, -1.0, kernel=k["id"], ws=ws, bias=bias, activation="relu", op_b="T")
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("with_ws", [False, True], ids=["no_ws", "ws"])
def test_skinny_nt_random_full_size(gpu_available, dtype, with_ws):
    """16 x 8192 x 8192 on N(0,1) data, the library's own choice: the error
    ratio of the untransposed paths, and bit-identical repeats."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=1110, dist="normal", dtype=dtype)
    Bt = B.t().contiguous()
    ws = nan_ws(M, N, K, dtype) if with_ws else None
    st, pl = plan(dtype, M, N, K, 0, nbytes(ws))
    name = tg.gemm_kernel_query(pl["kernel_id"])["name"]
    assert st == tg.GEMM_OK and "skinny_nt" in name, name
    say(f"[skinny nt] auto {name} M={M} N={N} K={K} random seed=1110 ws={with_ws}")
    C, _, _ = run_gemm(A, Bt, C0, 0.75, 0.5, ws=ws, op_b="T")
    if dtype == "fp8f32":
        r = layout_check(C, A, Bt, C0, 0.75, 0.5, "N", "T", dtype)
        say(f"[skinny nt] worst err/allowance {r:.3e}")
    else:
        a, b = host_view(A), host_view(Bt)
        ref = oracle.gemm_ref(a, b, 0.75, 0.5, C0.numpy(), "N", "T")
        D = oracle.gemm_absbound(a, b, 0.75, 0.5, C0.numpy(), "N", "T")
        r = oracle.error_ratio(C, ref, D)
        say(f"[skinny nt] ratio {r:.3e}")
        assert r <= TOL[dtype]
    Ad, Btd = to_dev(A), to_dev(Bt)
    outs = [tg.gemm(Ad, Btd, ws=ws, op_b="T") for _ in range(4)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    np.testing.assert_array_equal(outs[0].cpu().numpy(), tg.gemm(Ad, Btd, ws=ws, op_b="T").cpu().numpy())


@pytest.mark.parametrize("dtype", ALL)
def test_skinny_nt_split_matches_unsplit(gpu_available, dtype):
    """Few strips and a deep K: the workspace variant splits K across
    workgroups; both variants stay within the bound, and integer data gives
    identical results."""
    M, N, K = 16, 96, 16384
    ks = nt_kernels(dtype)
    plain = [k for n, k in ks.items() if "splitk" not in n][0]
    split = [k for n, k in ks.items() if "splitk" in n][0]
    ws = nan_ws(M, N, K, dtype)
    st, pl = plan(dtype, M, N, K, split["id"], nbytes(ws))
    assert st == tg.GEMM_OK and pl["grid"] == 3 * 8, pl
    A, B, C0 = make_integer_inputs(M, N, K, seed=1120, dtype=dtype)
    Bt = B.t().contiguous()
    say(f"[skinny nt] split vs plain M={M} N={N} K={K} seed=1120")
    C1, _, _ = run_gemm(A, Bt, C0, 1.0, 1.0, kernel=plain["id"], op_b="T")
    C2, _, _ = run_gemm(A, Bt, C0, 1.0, 1.0, kernel=split["id"], ws=ws, op_b="T")
    np.testing.assert_array_equal(C1, C2)
    np.testing.assert_array_equal(C1.astype(np.float64), ref_nt(A, Bt, C0, 1.0, 1.0))


@pytest.mark.parametrize("dtype", ALL)
def test_skinny_nt_padded_rows(gpu_available, dtype):
    """Padded leading dimensions (whole 16-byte chunks of NaN padding) on
    both operands: the padding is never read."""
    M, N, K = 7, 520, 2048
    chunk = 16 // ESZ[dtype]
    A, B, C0 = make_integer_inputs(M, N, K, seed=1130, dtype=dtype)
    Bt = B.t().contiguous()
    say(f"[skinny nt] padded M={M} N={N} K={K} pad={chunk} seed=1130")
    C, _, _ = run_gemm(A, Bt, C0, -1.0, 0.5, pad=(chunk, 2 * chunk, 0), op_b="T")
    np.testing.assert_array_equal(C.astype(np.float64), ref_nt(A, Bt, C0, -1.0, 0.5))


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
def test_skinny_nt_epilogue_random(gpu_available, dtype, act):
    """Every variant with the fused bias and activation on N(0,1) data, to
    the epilogue bound of the untransposed paths (the oracle takes the
    logical K x N operand)."""
    from test_epilogue import check_epilogue

    M, N, K = 11, 1000, 2048
    alpha = 1.0 / np.sqrt(K)
    A, B, C0 = make_random_inputs(M, N, K, seed=1140, dist="normal", dtype=dtype)
    Bt = B.t().contiguous()
    bias = make_bias(N, seed=1141)
    ws = nan_ws(M, N, K, dtype)
    for name, k in nt_kernels(dtype).items():
        say(f"[skinny nt] {name} M={M} N={N} K={K} act={act} random seed=1140")
        C, _, _ = run_gemm(A, Bt, C0, alpha, 0.5, kernel=k["id"], ws=ws, bias=bias, activation=act, op_b="T")
        if dtype == "fp8f32":
            r = layout_check(C, A, Bt, C0, alpha, 0.5, "N", "T", dtype, bias=bias, act=act)
        else:
            r = check_epilogue(C, A, B, C0, alpha, 0.5, bias, act, dtype)
        say(f"[skinny nt] worst err/allowance {r:.3e}")


def test_fp8_adversarial_runs_within_bound(gpu_available):
    """Every run of 8 consecutive k holds one product of 384 (256 x 1.5)
    among products of 2^-18 .. 2^-6 with mixed signs, so the matrix unit's
    truncation below 2^-13 of the run maximum drops most small products:
    every fp8 kernel for B stored N x K (skinny, ring, general) must stay
    within the run-truncation bound.  Values are exact E4M3 codes."""
    M, N, K = 16, 96, 1024
    rng = np.random.default_rng(1150)
    k = np.arange(K)
    big = (k % 8) == ((k // 8) * 3) % 8          # one position per run of 8
    tiny_a = rng.choice([2.0 ** -9, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6], size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    tiny_w = rng.choice([1.0, 0.5, 0.25, 2.0 ** -9], size=(N, K))
    A = np.where(big[None, :], 256.0, tiny_a).astype(np.float32)
    Wt = np.where(big[None, :], 1.5, tiny_w).astype(np.float32)
    A8 = torch.from_numpy(A).to(torch.float8_e4m3fn)
    W8 = torch.from_numpy(Wt).to(torch.float8_e4m3fn)
    assert torch.equal(A8.float(), torch.from_numpy(A)) and torch.equal(W8.float(), torch.from_numpy(Wt))
    C0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32))
    names = ["fp8_skinny_nt_n32_w8_u2", "fp8_mfma32_256x256x64_w2x2_nt_ring4", "fp8_general_128x128x16"]
    ids = {k["name"]: k["id"] for k in tg.kernels()}
    for name in names:
        say(f"[fp8 adversarial] {name} M={M} N={N} K={K} seed=1150")
        C, _, _ = run_gemm(A8, W8, C0, 1.0, 1.0, kernel=ids[name], op_b="T")
        r = layout_check(C, A8, W8, C0, 1.0, 1.0, "N", "T", "fp8f32")
        say(f"[fp8 adversarial] {name} worst err/allowance {r:.3e}")


# ----------------------------------------------------------------------------- both operands transposed

def tt_kernels(dtype):
    return {k["name"]: k for k in tg.kernels() if k["dtype"] == DT[dtype] and "skinny_tt" in k["name"]}


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("M", [1, 5, 12, 16])
@pytest.mark.parametrize("NK", [(8192, 4096), (1000, 3008), (33, 64)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_skinny_tt_exact(gpu_available, dtype, M, NK):
    """A stored K x M and B stored N x K: both forms forced and the library's
    choice with and without a workspace, with A's rows padded by 3 NaN
    elements (lda = M + 3) and A one element off alignment, bit-exact on
    integer data with bias and ReLU.  Columns past M must never reach C."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=1160 + M, dtype=dtype)
    As, Bt = A.t().contiguous(), B.t().contiguous()
    bias = make_bias(N, seed=1161, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(Bt), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu",
                                   "T", "T")
    ws = nan_ws(M, N, K, dtype)
    runs = [(n, k["id"], ws) for n, k in tt_kernels(dtype).items()] + [("auto", 0, None), ("auto ws", 0, ws)]
    for name, kid, w in runs:
        say(f"[skinny tt] {dtype} {name} M={M} N={N} K={K} lda={M + 3} offset=1 seed={1160 + M}")
        C, _, _ = run_gemm(As, Bt, C0, 2.0, -1.0, kernel=kid, ws=w, bias=bias, activation="relu", op_a="T",
                           op_b="T", pad=(3, 0, 0), offset=(1, 0, 0))
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)


@pytest.mark.parametrize("dtype", ALL)
@pytest.mark.parametrize("with_ws", [False, True], ids=["no_ws", "ws"])
def test_skinny_tt_random_matches_nt(gpu_available, dtype, with_ws):
    """12 x 8192 x 8192 on N(0,1) data through the forced both-transposed
    form: within the bound, and the same bits as the N x K kernel of the same
    form on A stored M x K (the same instruction inputs in the same order)."""
    M, N, K = 12, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=1170, dist="normal", dtype=dtype)
    As, Bt = A.t().contiguous(), B.t().contiguous()
    ws = nan_ws(M, N, K, dtype) if with_ws else None
    tt = {("splitk" in n): k["id"] for n, k in tt_kernels(dtype).items()}
    nt = {("splitk" in n): k["id"] for n, k in nt_kernels(dtype).items()}
    say(f"[skinny tt] {dtype} M={M} N={N} K={K} random seed=1170 ws={with_ws}")
    C, _, _ = run_gemm(As, Bt, C0, 0.75, 0.5, ws=ws, op_a="T", op_b="T", kernel=tt[with_ws])
    r = layout_check(C, As, Bt, C0, 0.75, 0.5, "T", "T", dtype)
    say(f"[skinny tt] worst err/allowance {r:.3e}")
    C2, _, _ = run_gemm(A, Bt, C0, 0.75, 0.5, ws=ws, op_b="T", kernel=nt[with_ws])
    np.testing.assert_array_equal(C, C2)
