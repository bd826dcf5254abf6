"""GPU parity of the fp8 skinny (M <= 16) kernels for weights stored K x N:
fp8 E4M3 weights streamed once through per-wave LDS rings, gathered with
byte-transposing reads, partials reduced in split order.

Integer operands make every sum exact (products of small integers, runs of
8 far below the truncation threshold), so results must equal the fp64
oracle bit for bit; random and adversarial operands check the fp8 kernels'
run-truncation bound.  Workspaces start full of NaN bit patterns."""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_integer_inputs, make_random_inputs

from gpu_helpers import host_view, run_gemm, say
from test_layouts import check as layout_check
from test_output_quant import run_quant

pytestmark = pytest.mark.gpu

FP8 = tg.GEMM_DTYPE_FP8F32
SPLIT = "fp8_skinny_kn_n128_w4_s4"
WHOLE = "fp8_skinny_kn_n128_w4_s4_whole_k"


def _ids():
    return {k["name"]: k["id"] for k in tg.kernels() if k["name"] in (SPLIT, WHOLE)}


def _ws(M, N, K):
    ws = tg.workspace(M, N, K, dtype=FP8)
    if ws is not None:
        ws.fill_(0xFF)
    return ws


def _plan(M, N, K, force=0, ws_bytes=0):
    return tg.gemm_plan_query_general(FP8, 0, 0, M, N, K, 1.0, 0x1000, K, 0x1000, N, -1.0, 0x1000, N, force,
                                      ws_bytes)


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("NK", [(8192, 8192), (4112, 8208), (1008, 3008)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fp8_kn_skinny_exact_both_variants(gpu_available, M, NK):
    """Both kernels, forced: N with a ragged last strip (4112 = 32 strips +
    16 columns, 1008), K with a partial last block (8208, 3008), M = 1, 5, 16;
    alpha, beta, bias and ReLU."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=1300 + M, dtype="fp8f32")
    bias = make_bias(N, seed=1301, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(A), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu")
    ws = _ws(M, N, K)
    for name, kid in _ids().items():
        st, pl = _plan(M, N, K, kid, ws.numel() if ws is not None else 0)
        assert st == tg.GEMM_OK, name
        say(f"[fp8 kn skinny] {name} M={M} N={N} K={K} grid={pl['grid']} splits={pl['splits']} exact relu "
            f"seed={1300 + M}")
        C, _, _ = run_gemm(A, B, C0, 2.0, -1.0, kernel=kid, ws=ws, bias=bias, activation="relu")
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)


def test_fp8_kn_skinny_random_and_deterministic(gpu_available):
    """The split form, forced, on 16 x 8192 x 8192 (64 strips x 4 splits):
    within the bound and bit-identical over five calls."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=1310, dist="normal", dtype="fp8f32")
    ws = _ws(M, N, K)
    kid = _ids()[SPLIT]
    st, pl = _plan(M, N, K, kid, ws.numel())
    assert st == tg.GEMM_OK and pl["grid"] == 256, pl
    say(f"[fp8 kn skinny] split M={M} N={N} K={K} random seed=1310")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=ws, kernel=kid)
    r = layout_check(C, A, B, C0, 1.0, 0.5, "N", "N", "fp8f32")
    say(f"[fp8 kn skinny] worst err/allowance {r:.3e}")
    Ad, Bd = A.cuda(), B.cuda()
    outs = [tg.gemm(Ad, Bd, ws=ws, kernel=kid) for _ in range(5)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_fp8_kn_skinny_without_workspace(gpu_available):
    """16 x 8192 x 8192 without a workspace: the kernel over the whole of K
    (64 workgroups), within the bound and bit-identical on repeats."""
    M, N, K = 16, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=1311, dist="normal", dtype="fp8f32")
    st, pl = _plan(M, N, K)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] == WHOLE and pl["grid"] == 64, pl
    say(f"[fp8 kn skinny] auto, no workspace M={M} N={N} K={K} random seed=1311")
    C, _, _ = run_gemm(A, B, C0, 1.0, 0.5)
    r = layout_check(C, A, B, C0, 1.0, 0.5, "N", "N", "fp8f32")
    say(f"[fp8 kn skinny] worst err/allowance {r:.3e}")
    Ad, Bd = A.cuda(), B.cuda()
    outs = [tg.gemm(Ad, Bd) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_fp8_kn_skinny_adversarial_runs(gpu_available):
    """Every run of 8 consecutive k holds one product of 384 among products
    of 2^-18 .. 2^-6 with mixed signs (the matrix unit truncates below 2^-13
    of the run maximum): both kernels stay within the run-truncation bound.
    Values are exact E4M3 codes."""
    M, N, K = 16, 272, 1088
    rng = np.random.default_rng(1312)
    k = np.arange(K)
    big = (k % 8) == ((k // 8) * 5) % 8          # one position per run of 8
    tiny_a = rng.choice([2.0 ** -9, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6], size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    tiny_b = rng.choice([1.0, 0.5, 0.25, 2.0 ** -9], size=(K, N))
    A = np.where(big[None, :], 256.0, tiny_a).astype(np.float32)
    B = np.where(big[:, None], 1.5, tiny_b).astype(np.float32)
    A8 = torch.from_numpy(A).to(torch.float8_e4m3fn)
    B8 = torch.from_numpy(B).to(torch.float8_e4m3fn)
    assert torch.equal(A8.float(), torch.from_numpy(A)) and torch.equal(B8.float(), torch.from_numpy(B))
    C0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32))
    ws = _ws(M, N, K)
    for name, kid in _ids().items():
        say(f"[fp8 kn adversarial] {name} M={M} N={N} K={K} seed=1312")
        C, _, _ = run_gemm(A8, B8, C0, 1.0, 1.0, kernel=kid, ws=ws)
        r = layout_check(C, A8, B8, C0, 1.0, 1.0, "N", "N", "fp8f32")
        say(f"[fp8 kn adversarial] {name} worst err/allowance {r:.3e}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fp8_kn_skinny_quantised_output(gpu_available, kind):
    """bf16 and E4M3 outputs (scale 1/4) with beta, bias and ReLU, exact on
    integer data, through both kernels (the split one through the reduce)."""
    M, N, K = 13, 1008, 3008
    A, B, C0 = make_integer_inputs(M, N, K, seed=1313, dtype="fp8f32")
    bias = make_bias(N, seed=1314, integer=True)
    z = oracle.gemm_epilogue_ref(host_view(A), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu")
    ws = _ws(M, N, K)
    for name, kid in _ids().items():
        say(f"[fp8 kn skinny] {name} -> {kind} M={M} N={N} K={K} seed=1313")
        got = run_quant(A, B, C0, 2.0, -1.0, kind, 0.25, kernel=kid, ws=ws, bias=bias, act="relu")
        np.testing.assert_array_equal(got, oracle.quantize(z, kind, 0.25), err_msg=name)


AT_SPLIT = "fp8_skinny_kn_at1_n128_w4_s3"
AT_WHOLE = "fp8_skinny_kn_at1_n128_w4_s3_whole_k"


def _at_ids():
    return {k["name"]: k["id"] for k in tg.kernels() if k["name"] in (AT_SPLIT, AT_WHOLE)}


@pytest.mark.parametrize("M", [1, 5, 12, 16])
@pytest.mark.parametrize("NK", [(8192, 4096), (1008, 3008), (4112, 8208)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_fp8_kn_skinny_a_transposed_exact(gpu_available, M, NK):
    """A stored K x M, loaded a byte a lane (any M): both forms forced and
    the library's choice with and without a workspace, with A's rows padded
    by 3 NaN bytes and A one byte off alignment (so the 128^2 ring cannot
    run), bit-exact on integer data with bias and ReLU.  Columns past M must
    never reach C; rows past K must read as zero."""
    N, K = NK
    A, B, C0 = make_integer_inputs(M, N, K, seed=1320 + M, dtype="fp8f32")
    As = A.t().contiguous()
    bias = make_bias(N, seed=1321, integer=True)
    ref = oracle.gemm_epilogue_ref(host_view(As), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu", "T", "N")
    ws = _ws(M, N, K)
    runs = [(n, kid, ws) for n, kid in _at_ids().items()] + [("auto", 0, None), ("auto ws", 0, ws)]
    for name, kid, w in runs:
        say(f"[fp8 kn skinny A^T] {name} M={M} N={N} K={K} lda={M + 3} offset=1 seed={1320 + M}")
        C, _, _ = run_gemm(As, B, C0, 2.0, -1.0, kernel=kid, ws=w, bias=bias, activation="relu", op_a="T",
                           pad=(3, 0, 0), offset=(1, 0, 0))
        np.testing.assert_array_equal(C.astype(np.float64), ref, err_msg=name)
    st, pl = tg.gemm_plan_query_general(FP8, 1, 0, M, N, K, 1.0, 0x1001, M + 3, 0x1000, N, 0.0, 0x1000, N, 0, 0)
    assert st == tg.GEMM_OK and tg.gemm_kernel_query(pl["kernel_id"])["name"] == AT_WHOLE, pl


def test_fp8_kn_skinny_a_transposed_random(gpu_available):
    """12 x 8192 x 8192, A stored K x 12 (N(0,1) bytes), with and without a
    workspace: within the run-truncation bound, and the same bits as the
    untransposed kernel of the same form (the same instruction inputs in the
    same order)."""
    M, N, K = 12, 8192, 8192
    A, B, C0 = make_random_inputs(M, N, K, seed=1322, dist="normal", dtype="fp8f32")
    As = A.t().contiguous()
    ws = _ws(M, N, K)
    at, nn = _at_ids(), _ids()
    for w, at_name, nn_name in [(ws, AT_SPLIT, SPLIT), (None, AT_WHOLE, WHOLE)]:
        say(f"[fp8 kn skinny A^T] {at_name} M={M} N={N} K={K} normal seed=1322")
        C, _, _ = run_gemm(As, B, C0, 1.0, 0.5, ws=w, op_a="T", kernel=at[at_name])
        r = layout_check(C, As, B, C0, 1.0, 0.5, "T", "N", "fp8f32")
        say(f"[fp8 kn skinny A^T] worst err/allowance {r:.3e}")
        C2, _, _ = run_gemm(A, B, C0, 1.0, 0.5, ws=w, kernel=nn[nn_name])
        np.testing.assert_array_equal(C, C2)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fp8_kn_skinny_a_transposed_quantised_output(gpu_available, kind):
    """A stored K x 13 (rows of 13 bytes, which only the byte-loading form
    runs): bf16 and E4M3 outputs (scale 1/4, output rows padded by 3) with
    beta, bias and ReLU, exact on integer data, through both forms."""
    M, N, K = 13, 1008, 3008
    A, B, C0 = make_integer_inputs(M, N, K, seed=1323, dtype="fp8f32")
    As = A.t().contiguous()
    bias = make_bias(N, seed=1324, integer=True)
    z = oracle.gemm_epilogue_ref(host_view(As), host_view(B), 2.0, -1.0, C0.numpy(), bias.numpy(), "relu", "T", "N")
    ws = _ws(M, N, K)
    for name, kid in _at_ids().items():
        say(f"[fp8 kn skinny A^T] {name} -> {kind} M={M} N={N} K={K} seed=1323")
        got = run_quant(As, B, C0, 2.0, -1.0, kind, 0.25, kernel=kid, ws=ws, bias=bias, act="relu", op_a="T", pad=3)
        np.testing.assert_array_equal(got, oracle.quantize(z, kind, 0.25), err_msg=name)
