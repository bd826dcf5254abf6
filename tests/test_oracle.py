"""Pins for the fp64 CPU oracle.

The oracle computes C = alpha*(A x B) + beta*C0 (the defining formula of "GEMM
Worklog I: Naive to Tiled" and the one-call problem of "A GEMM Kernel, Step by
Step").  Nothing here re-types that formula: each test checks the oracle
against something fixed independently of it -- a closed form for a special
operand (identity, permutation, all-ones, rank one), exact rational brute
force, a library routine (torch's fp64 matmul), algebraic invariants, or the
bf16 format definition.  A planted mistake in the oracle (dropped term, wrong
sign, wrong index, transposed operand, ignored leading dimension) fails at
least one of them; tests/test_oracle_mutants.py proves that by building such
mutants.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -53  # fp64 unit roundoff


def rand32(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def padded(x: np.ndarray, extra: int, fill=np.nan) -> np.ndarray:
    """View of x inside a wider buffer whose padding columns hold ``fill``."""
    rows, cols = x.shape
    buf = np.full((rows, cols + extra), fill, dtype=x.dtype)
    buf[:, :cols] = x
    return buf[:, :cols]


def exact_gemm(A, B, alpha, beta, C0):
    """Exact rational value of every entry (tiny shapes only)."""
    M, K = A.shape
    N = B.shape[1]
    fa, fb = Fraction(float(alpha)), Fraction(float(beta))
    out = np.empty((M, N), dtype=object)
    bnd = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                p = Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                s += p
                sa += abs(p)
            v = fa * s
            d = abs(fa) * sa
            if beta != 0.0:
                c = Fraction(float(C0[i, j]))
                v += fb * c
                d += abs(fb) * abs(c)
            out[i, j] = v
            bnd[i, j] = d
    return out, bnd


SHAPES_TINY = [(1, 1, 1), (1, 5, 3), (7, 1, 4), (3, 4, 1), (8, 8, 8), (5, 3, 7), (2, 6, 5), (4, 4, 0)]
SCALARS = [(1.0, 0.0), (2.0, -1.0), (-0.75, 0.5), (0.0, 1.5), (1.0, 1.0)]


# ----------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("M", [1, 5, 33])
@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_identity_left(M, alpha, beta):
    """A = I gives C = alpha*B + beta*C0: one exact product per entry, then the scalars."""
    rng = np.random.default_rng(10 + M)
    N = 19
    A = np.eye(M, dtype=np.float32)
    B = rand32(rng, (M, N))
    C0 = rand32(rng, (M, N))
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    want = alpha * B.astype(np.float64)
    if beta != 0.0:
        want = want + beta * C0.astype(np.float64)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_identity_right(alpha, beta):
    """B = I gives C = alpha*A + beta*C0."""
    rng = np.random.default_rng(3)
    M, K = 23, 17
    A = rand32(rng, (M, K))
    B = np.eye(K, dtype=np.float32)
    C0 = rand32(rng, (M, K))
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    want = alpha * A.astype(np.float64)
    if beta != 0.0:
        want = want + beta * C0.astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_permutation_left_selects_rows_of_B():
    """A = row-selection matrix: row i of C is row perm[i] of B (scaled)."""
    rng = np.random.default_rng(4)
    M, K, N = 13, 29, 11
    perm = rng.integers(0, K, size=M)
    A = np.zeros((M, K), dtype=np.float32)
    A[np.arange(M), perm] = 1.0
    B = rand32(rng, (K, N))
    C0 = rand32(rng, (M, N))
    got = oracle.gemm_ref(A, B, 2.0, -1.0, C0)
    want = 2.0 * B[perm].astype(np.float64) - C0.astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_permutation_right_selects_columns_of_A():
    """B = column-selection matrix: column j of C is column q[j] of A."""
    rng = np.random.default_rng(5)
    M, K, N = 9, 21, 14
    q = rng.permutation(K)[:N]
    B = np.zeros((K, N), dtype=np.float32)
    B[q, np.arange(N)] = 1.0
    A = rand32(rng, (M, K))
    got = oracle.gemm_ref(A, B, 0.5, 0.0)
    want = 0.5 * A[:, q].astype(np.float64)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (16, 8, 1000), (1, 1, 4097)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (2.0, -1.0), (-3.0, 0.25)])
def test_all_ones(M, N, K, alpha, beta):
    """All-ones A and B: every entry is alpha*K + beta*C0 exactly."""
    rng = np.random.default_rng(M * 7 + K)
    A = np.ones((M, K), dtype=np.float32)
    B = np.ones((K, N), dtype=np.float32)
    C0 = rand32(rng, (M, N))
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    want = np.full((M, N), alpha * K, dtype=np.float64)
    if beta != 0.0:
        want = want + beta * C0.astype(np.float64)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_rank_one(alpha, beta):
    """K = 1: C is the scaled outer product of the single column and row."""
    rng = np.random.default_rng(6)
    M, N = 17, 12
    A = rand32(rng, (M, 1))
    B = rand32(rng, (1, N))
    C0 = rand32(rng, (M, N))
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    want = alpha * np.multiply.outer(A[:, 0].astype(np.float64), B[0].astype(np.float64))
    if beta != 0.0:
        want = want + beta * C0.astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_k_zero_is_empty_sum():
    """K = 0: the sum is empty, C = beta*C0 (or 0)."""
    C0 = np.arange(12, dtype=np.float32).reshape(3, 4)
    A = np.zeros((3, 0), dtype=np.float32)
    B = np.zeros((0, 4), dtype=np.float32)
    np.testing.assert_array_equal(oracle.gemm_ref(A, B, 2.0, 0.5, C0), 0.5 * C0.astype(np.float64))
    np.testing.assert_array_equal(oracle.gemm_ref(A, B, 2.0, 0.0, C0), np.zeros((3, 4)))


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("shape", SHAPES_TINY)
@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_bruteforce_dyadic_exact(shape, alpha, beta):
    """Small dyadic operands: every partial sum is exact, so the oracle must equal
    the exact rational result computed term by term."""
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = (rng.integers(-8, 9, size=(M, K)) / 4.0).astype(np.float32)
    B = (rng.integers(-8, 9, size=(K, N)) / 8.0).astype(np.float32)
    C0 = (rng.integers(-8, 9, size=(M, N)) / 2.0).astype(np.float32)
    exact, _ = exact_gemm(A, B, alpha, beta, C0)
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    want = np.array([[float(v) for v in row] for row in exact], dtype=np.float64).reshape(M, N)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("shape", SHAPES_TINY)
@pytest.mark.parametrize("alpha,beta", SCALARS)
def test_bruteforce_random_within_fp64_bound(shape, alpha, beta):
    """Random fp32 operands: the oracle sits within (K+2)*u*D of the exact value,
    the forward error bound of an fp64 inner product of exact terms."""
    M, N, K = shape
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    A, B, C0 = rand32(rng, (M, K)), rand32(rng, (K, N)), rand32(rng, (M, N))
    exact, bnd = exact_gemm(A, B, alpha, beta, C0)
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(got[i, j])) - exact[i, j])
            assert err <= Fraction(K + 2) * Fraction(U) * bnd[i, j], (i, j)


# ----------------------------------------------------------------------------- library routine

@pytest.mark.parametrize("M,N,K", [(64, 96, 200), (300, 200, 500), (1, 257, 129), (33, 1, 65)])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (2.0, -1.0), (1.0, 0.5)])
def test_matches_torch_float64_matmul(M, N, K, alpha, beta):
    """torch's double-precision matmul (a BLAS dgemm) agrees within 2*(K+2)*u*D."""
    rng = np.random.default_rng(M + N + K)
    A, B, C0 = rand32(rng, (M, K)), rand32(rng, (K, N)), rand32(rng, (M, N))
    got = oracle.gemm_ref(A, B, alpha, beta, C0)
    t = alpha * (torch.from_numpy(A).double() @ torch.from_numpy(B).double())
    if beta != 0.0:
        t = t + beta * torch.from_numpy(C0).double()
    D = oracle.gemm_absbound(A, B, alpha, beta, C0)
    assert np.all(np.abs(got - t.numpy()) <= 2 * (K + 2) * U * D)


# ----------------------------------------------------------------------------- invariants

def test_transpose_invariant():
    """(A B)^T = B^T A^T term by term, in the same k order, so bitwise."""
    rng = np.random.default_rng(7)
    M, N, K = 37, 23, 51
    A, B, C0 = rand32(rng, (M, K)), rand32(rng, (K, N)), rand32(rng, (M, N))
    C = oracle.gemm_ref(A, B, 1.5, -0.5, C0)
    Ct = oracle.gemm_ref(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), 1.5, -0.5,
                         np.ascontiguousarray(C0.T))
    np.testing.assert_array_equal(C, Ct.T)


def test_not_symmetric_in_operands():
    """Swapping A and B (square case) changes the answer: guards against an
    oracle that accidentally computes B A or A^T B."""
    rng = np.random.default_rng(8)
    A, B = rand32(rng, (8, 8)), rand32(rng, (8, 8))
    assert not np.allclose(oracle.gemm_ref(A, B), oracle.gemm_ref(B, A))
    assert not np.allclose(oracle.gemm_ref(A, B), oracle.gemm_ref(np.ascontiguousarray(A.T), B))


@pytest.mark.parametrize("p", [-3, 1, 5])
def test_alpha_power_of_two_scales_exactly(p):
    rng = np.random.default_rng(9)
    A, B = rand32(rng, (11, 30)), rand32(rng, (30, 13))
    np.testing.assert_array_equal(oracle.gemm_ref(A, B, 2.0 ** p), (2.0 ** p) * oracle.gemm_ref(A, B, 1.0))


def test_alpha_sign_flips():
    rng = np.random.default_rng(19)
    A, B = rand32(rng, (11, 30)), rand32(rng, (30, 13))
    np.testing.assert_array_equal(oracle.gemm_ref(A, B, -1.0), -oracle.gemm_ref(A, B, 1.0))


def test_beta_term_is_linear_in_C0():
    """C(beta, C0) - C(0) = beta*C0 up to one rounding per entry."""
    rng = np.random.default_rng(20)
    A, B, C0 = rand32(rng, (9, 40)), rand32(rng, (40, 7)), rand32(rng, (9, 7))
    diff = oracle.gemm_ref(A, B, 1.0, 0.75, C0) - oracle.gemm_ref(A, B, 1.0, 0.0)
    D = oracle.gemm_absbound(A, B, 1.0, 0.75, C0)
    assert np.all(np.abs(diff - 0.75 * C0.astype(np.float64)) <= 4 * U * D)


def test_k_split_additivity():
    """A B = A[:, :k] B[:k] + A[:, k:] B[k:] within fp64 rounding."""
    rng = np.random.default_rng(11)
    M, N, K, k1 = 19, 17, 90, 37
    A, B = rand32(rng, (M, K)), rand32(rng, (K, N))
    full = oracle.gemm_ref(A, B)
    part = (oracle.gemm_ref(np.ascontiguousarray(A[:, :k1]), np.ascontiguousarray(B[:k1]))
            + oracle.gemm_ref(np.ascontiguousarray(A[:, k1:]), np.ascontiguousarray(B[k1:])))
    D = oracle.gemm_absbound(A, B)
    assert np.all(np.abs(full - part) <= 2 * (K + 2) * U * D)
    assert not np.array_equal(oracle.gemm_ref(np.ascontiguousarray(A[:, :k1]),
                                              np.ascontiguousarray(B[:k1])), full)


# ----------------------------------------------------------------------------- conventions

def test_beta_zero_does_not_read_C0():
    """beta == 0 leaves the C0 term out entirely, so NaN in C0 cannot appear."""
    rng = np.random.default_rng(12)
    A, B = rand32(rng, (6, 9)), rand32(rng, (9, 5))
    C0 = np.full((6, 5), np.nan, dtype=np.float32)
    got = oracle.gemm_ref(A, B, 1.0, 0.0, C0)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got, oracle.gemm_ref(A, B, 1.0, 0.0, None))


def test_beta_nonzero_propagates_nan_per_entry():
    rng = np.random.default_rng(13)
    A, B = rand32(rng, (6, 9)), rand32(rng, (9, 5))
    C0 = rand32(rng, (6, 5))
    C0[2, 3] = np.nan
    got = oracle.gemm_ref(A, B, 1.0, 1.0, C0)
    assert np.isnan(got[2, 3])
    assert np.isfinite(np.delete(got.ravel(), 2 * 5 + 3)).all()


@pytest.mark.parametrize("pa,pb,pc", [(3, 0, 0), (0, 5, 0), (0, 0, 7), (1, 2, 3)])
def test_leading_dimensions_honoured(pa, pb, pc):
    """Views into NaN-padded buffers give the same result as packed copies."""
    rng = np.random.default_rng(14)
    M, N, K = 10, 12, 9
    A, B, C0 = rand32(rng, (M, K)), rand32(rng, (K, N)), rand32(rng, (M, N))
    want = oracle.gemm_ref(A, B, 2.0, -1.0, C0)
    got = oracle.gemm_ref(padded(A, pa), padded(B, pb), 2.0, -1.0, padded(C0, pc))
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- bf16 operands

BF16_BITS = {
    0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F81: 1.0 + 2.0 ** -7,
    0x3E80: 0.25, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,   # largest finite bf16
    0x0080: 2.0 ** -126,                                    # smallest normal
    0x0001: 2.0 ** -133,                                    # smallest subnormal
    0x8000: -0.0, 0x4049: 3.140625,
}


@pytest.mark.parametrize("bits,value", sorted(BF16_BITS.items()))
def test_bf16_widening_follows_format(bits, value):
    """A 1x1x1 product with B = 1.0 returns the operand's value as the bf16
    format defines it (sign, 8-bit exponent, 7-bit fraction)."""
    A = np.array([[bits]], dtype=np.uint16)
    one = np.array([[0x3F80]], dtype=np.uint16)
    got = oracle.gemm_ref(A, one)[0, 0]
    assert got == value   # -0.0 sums to +0.0 from the empty-sum start; equal as values
    got_b = oracle.gemm_ref(one, A)[0, 0]
    assert got_b == value


def test_bf16_matches_f32_path_on_same_values():
    """bf16 operands widened by the format give the same fp64 result as the same
    values handed over as fp32 (torch's bf16 -> fp32 conversion is exact)."""
    g = torch.Generator().manual_seed(15)
    A = torch.randn(21, 44, generator=g).to(torch.bfloat16)
    B = torch.randn(44, 18, generator=g).to(torch.bfloat16)
    C0 = torch.randn(21, 18, generator=g)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    got = oracle.gemm_ref(bits(A), bits(B), 1.0, 0.5, C0.numpy())
    want = oracle.gemm_ref(A.float().numpy(), B.float().numpy(), 1.0, 0.5, C0.numpy())
    np.testing.assert_array_equal(got, want)
    Db = oracle.gemm_absbound(bits(A), bits(B), 1.0, 0.5, C0.numpy())
    Df = oracle.gemm_absbound(A.float().numpy(), B.float().numpy(), 1.0, 0.5, C0.numpy())
    np.testing.assert_array_equal(Db, Df)


def test_bf16_identity():
    g = torch.Generator().manual_seed(16)
    B = torch.randn(8, 9, generator=g).to(torch.bfloat16)
    I = torch.eye(8).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.gemm_ref(bits(I), bits(B), 3.0),
                                  3.0 * B.double().numpy())


# ----------------------------------------------------------------------------- denominator

def test_absbound_all_ones():
    C0 = np.array([[-2.0, 3.0]], dtype=np.float32)
    A = -np.ones((1, 5), dtype=np.float32)
    B = np.ones((5, 2), dtype=np.float32)
    np.testing.assert_array_equal(oracle.gemm_absbound(A, B, -2.0, -0.5, C0),
                                  np.array([[10.0 + 1.0, 10.0 + 1.5]]))


def test_absbound_identity_and_sign_invariance():
    rng = np.random.default_rng(17)
    B, C0 = rand32(rng, (6, 4)), rand32(rng, (6, 4))
    I = np.eye(6, dtype=np.float32)
    D = oracle.gemm_absbound(I, B, -2.0, 0.5, C0)
    np.testing.assert_array_equal(D, 2.0 * np.abs(B.astype(np.float64)) + 0.5 * np.abs(C0.astype(np.float64)))
    A, C1 = rand32(rng, (5, 6)), rand32(rng, (5, 4))
    np.testing.assert_array_equal(oracle.gemm_absbound(A, B, 1.0, 0.5, C1),
                                  oracle.gemm_absbound(-A, B, -1.0, -0.5, -C1))


def test_absbound_dominates_result_and_equals_gemm_of_abs():
    """|C| <= D by the triangle inequality, and D is the GEMM of the absolute values."""
    rng = np.random.default_rng(18)
    A, B, C0 = rand32(rng, (12, 33)), rand32(rng, (33, 10)), rand32(rng, (12, 10))
    C = oracle.gemm_ref(A, B, -1.5, 0.25, C0)
    D = oracle.gemm_absbound(A, B, -1.5, 0.25, C0)
    assert np.all(np.abs(C) <= D * (1 + 64 * U))
    np.testing.assert_array_equal(D, oracle.gemm_ref(np.abs(A), np.abs(B), 1.5, 0.25, np.abs(C0)))


# ----------------------------------------------------------------------------- fp8 (OCP E4M3) operands

# Code -> value from the E4M3 definition (bias 7; exponent field 0 subnormal
# m * 2^-9; S.1111.111 NaN; no infinities).
E4M3_TABLE = [(0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
              (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
              (0xFE, -448.0), (0xB8, -1.0), (0x77, 240.0), (0x7F, np.nan), (0xFF, np.nan)]


@pytest.mark.parametrize("code,value", E4M3_TABLE)
def test_fp8_widening_follows_format(code, value):
    one = np.uint8([[0x38]])
    got = oracle.gemm_ref(np.uint8([[code]]), one)[0, 0]
    if np.isnan(value):
        assert np.isnan(got)
    else:
        assert got == value          # a sum starts at +0, so the sign of -0 is not kept


def test_fp8_every_code_matches_torch_decode():
    """All 256 codes against torch's float8_e4m3fn decode (independent code)."""
    codes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = oracle.gemm_ref(codes, np.uint8([[0x38]]))[:, 0]
    ref = torch.from_numpy(codes[:, 0].copy()).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(got, ref)


def test_fp8_matches_f32_path_on_same_values():
    rng = np.random.default_rng(30)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    A = rng.choice(codes, size=(9, 37)).astype(np.uint8)
    B = rng.choice(codes, size=(37, 11)).astype(np.uint8)
    C0 = rand32(rng, (9, 11))
    to32 = lambda x: torch.from_numpy(x).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(oracle.gemm_ref(A, B, -0.5, 2.0, C0),
                                  oracle.gemm_ref(to32(A), to32(B), -0.5, 2.0, C0))
    np.testing.assert_array_equal(oracle.gemm_absbound(A, B, -0.5, 2.0, C0),
                                  oracle.gemm_absbound(to32(A), to32(B), -0.5, 2.0, C0))


def test_fp8_identity():
    rng = np.random.default_rng(31)
    B = rng.integers(0, 256, size=(6, 7)).astype(np.uint8)
    B[B == 0x7F] = 0x38
    B[B == 0xFF] = 0xB8
    eye = np.where(np.eye(6, dtype=bool), 0x38, 0x00).astype(np.uint8)
    vals = torch.from_numpy(B).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(oracle.gemm_ref(eye, B, 2.0), 2.0 * vals)


@pytest.mark.parametrize("pa,pb,pc", [(3, 0, 0), (0, 5, 0), (0, 0, 7), (1, 2, 3)])
def test_fp8_leading_dimensions_honoured(pa, pb, pc):
    """fp8 views into padded buffers (padding bytes 0x7F, NaN) equal packed copies."""
    rng = np.random.default_rng(34)
    M, N, K = 10, 12, 9
    A = rng.integers(0, 0x7E, size=(M, K)).astype(np.uint8)
    B = rng.integers(0x80, 0xFE, size=(K, N)).astype(np.uint8)
    C0 = rand32(rng, (M, N))
    want = oracle.gemm_ref(A, B, 2.0, -1.0, C0)
    got = oracle.gemm_ref(padded(A, pa, 0x7F), padded(B, pb, 0x7F), 2.0, -1.0, padded(C0, pc))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(oracle.gemm_groupmax(padded(A, pa, 0x7F), padded(B, pb, 0x7F), 2.0),
                                  oracle.gemm_groupmax(A, B, 2.0))


# ----------------------------------------------------------------------------- operand layouts

@pytest.mark.parametrize("dt", [np.float32, np.uint16, np.uint8])
def test_transposed_layouts_multiply_the_transpose(dt):
    """op(X) = X^T: passing A^T with op_a = "T" (and B^T with op_b = "T")
    gives the plain product; and C^T = B^T A^T swaps the roles."""
    rng = np.random.default_rng(32)
    if dt == np.float32:
        A, B = rand32(rng, (5, 9)), rand32(rng, (9, 4))
    else:
        A = rng.integers(0, 0x3F, size=(5, 9)).astype(dt)      # finite, positive codes
        B = rng.integers(0, 0x3F, size=(9, 4)).astype(dt)
    ref = oracle.gemm_ref(A, B, 1.5)
    At, Bt = np.ascontiguousarray(A.T), np.ascontiguousarray(B.T)
    np.testing.assert_array_equal(oracle.gemm_ref(At, B, 1.5, op_a="T"), ref)
    np.testing.assert_array_equal(oracle.gemm_ref(A, Bt, 1.5, op_b="T"), ref)
    np.testing.assert_array_equal(oracle.gemm_ref(At, Bt, 1.5, op_a="T", op_b="T"), ref)
    np.testing.assert_array_equal(oracle.gemm_ref(B, A, 1.5, op_a="T", op_b="T"), ref.T)
    with pytest.raises(ValueError):
        oracle.gemm_ref(A, B, op_a="X")


# ----------------------------------------------------------------------------- fp8 group bound

@pytest.mark.parametrize("K", [1, 7, 8, 9, 64, 70])
def test_groupmax_all_ones_counts_runs(K):
    ones_a = np.full((3, K), 0x38, np.uint8)
    ones_b = np.full((K, 5), 0x38, np.uint8)
    np.testing.assert_array_equal(oracle.gemm_groupmax(ones_a, ones_b, -2.0), np.full((3, 5), 2.0 * -(-K // 8)))


def test_groupmax_bruteforce():
    rng = np.random.default_rng(33)
    A = rng.integers(0, 0x7E, size=(4, 21)).astype(np.uint8) | (rng.integers(0, 2, size=(4, 21)) << 7).astype(np.uint8)
    B = rng.integers(0, 0x7E, size=(21, 3)).astype(np.uint8)
    a = torch.from_numpy(A).view(torch.float8_e4m3fn).double().numpy()
    b = torch.from_numpy(B).view(torch.float8_e4m3fn).double().numpy()
    G = oracle.gemm_groupmax(A, B, 0.5)
    for i in range(4):
        for j in range(3):
            expect = sum(max(abs(a[i, k] * b[k, j]) for k in range(q, min(q + 8, 21))) for q in range(0, 21, 8))
            assert G[i, j] == 0.5 * expect
    D = oracle.gemm_absbound(A, B, 0.5)
    assert np.all(G <= D) and np.all(8 * G >= D)


# ----------------------------------------------------------------------------- fused epilogue
# act(Z + bias) on a finished GEMM result ("Tiled matrix multiplication",
# "Efficiency" and "Implementation notes").  ReLU and GELU are pinned by
# closed forms, normal-table values, the identity Phi(x) + Phi(-x) = 1 and
# scipy's normal CDF (the Cephes ndtr, code independent of the C library's
# erf that the oracle calls).

PHI_1 = 0.8413447460685429          # standard normal CDF at 1 (normal tables)
Z975 = 1.959963984540054            # the 97.5% quantile of the standard normal


def test_epilogue_none_is_identity():
    Z = np.array([[-3.0, -0.0, 0.0, 2.5, np.inf, -np.inf, np.nan]])
    out = oracle.epilogue_ref(Z)
    np.testing.assert_array_equal(out, Z)
    assert np.signbit(out[0, 1]) and not np.signbit(out[0, 2])


def test_relu_closed_forms():
    Z = np.array([[-3.0, -1e-300, 0.0, 2.5, 1e300, np.inf, -np.inf, np.nan]])
    out = oracle.epilogue_ref(Z, activation="relu")
    np.testing.assert_array_equal(out, [[0.0, 0.0, 0.0, 2.5, 1e300, np.inf, 0.0, np.nan]])


def test_relu_splits_into_positive_and_negative_parts():
    rng = np.random.default_rng(40)
    x = rng.normal(size=(7, 9))
    pos = oracle.epilogue_ref(x, activation="relu")
    neg = oracle.epilogue_ref(-x, activation="relu")
    np.testing.assert_array_equal(pos - neg, x)            # x = x+ - x-
    np.testing.assert_array_equal(pos * neg, np.zeros_like(x))
    assert np.all(pos >= 0)


def test_gelu_table_values():
    Z = np.array([[0.0, 1.0, -1.0, Z975, -Z975, 10.0]])
    out = oracle.epilogue_ref(Z, activation="gelu")[0]
    assert out[0] == 0.0
    assert abs(out[1] - PHI_1) <= 4 * U
    assert abs(out[2] - (-(1.0 - PHI_1))) <= 4 * U
    assert abs(out[3] - Z975 * 0.975) <= 8 * U
    assert abs(out[4] - (-Z975 * 0.025)) <= 8 * U
    assert out[5] == 10.0                                   # 1 - Phi(10) < 1e-23


def test_gelu_odd_part_is_identity():
    """gelu(x) - gelu(-x) = x (Phi(x) + Phi(-x) = 1), and gelu(x) + gelu(-x) = x*(2*Phi(x) - 1) >= 0."""
    rng = np.random.default_rng(41)
    x = rng.normal(scale=3.0, size=(11, 13))
    g = oracle.epilogue_ref(x, activation="gelu")
    gm = oracle.epilogue_ref(-x, activation="gelu")
    np.testing.assert_allclose(g - gm, x, rtol=4 * U, atol=4 * U)
    assert np.all(g + gm >= -4 * U)


def test_gelu_matches_scipy_normal_cdf():
    """The erf form 1 + erf(x/sqrt 2) cancels in the left tail, so the
    agreement is absolute, a few ulps of |x|, not relative."""
    from scipy.special import ndtr
    x = np.linspace(-8.0, 8.0, 321).reshape(3, 107)
    g = oracle.epilogue_ref(x, activation="gelu")
    assert np.all(np.abs(g - x * ndtr(x)) <= 8 * U * np.abs(x))
    right = x > 0.5
    np.testing.assert_allclose(g[right], (x * ndtr(x))[right], rtol=1e-14)


def test_gelu_tails_and_special_values():
    out = oracle.epilogue_ref(np.array([[-10.0, 40.0, np.inf, np.nan]]), activation="gelu")[0]
    assert -1e-20 < out[0] <= 0.0                         # 1 + erf(-10/sqrt 2) rounds to 0
    assert out[1] == 40.0 and out[2] == np.inf and np.isnan(out[3])


def test_bias_is_indexed_by_column():
    bias = np.float32([1.0, -2.0, 3.5, 0.25, -0.125])
    out = oracle.epilogue_ref(np.zeros((7, 5)), bias)
    np.testing.assert_array_equal(out, np.tile(bias.astype(np.float64), (7, 1)))


def test_bias_with_identity_operand():
    """act(I @ B + bias) with small integers: B + bias exactly, then the activation."""
    rng = np.random.default_rng(42)
    B = rng.integers(-5, 6, size=(6, 9)).astype(np.float32)
    bias = rng.integers(-3, 4, size=9).astype(np.float32)
    eye = np.eye(6, dtype=np.float32)
    np.testing.assert_array_equal(oracle.gemm_epilogue_ref(eye, B, bias=bias), B + bias)
    np.testing.assert_array_equal(oracle.gemm_epilogue_ref(eye, B, bias=bias, activation="relu"),
                                  np.maximum(B + bias, 0.0))
    np.testing.assert_array_equal(oracle.gemm_epilogue_ref(eye, B, 2.0, 0.0, None, bias),
                                  2.0 * B.astype(np.float64) + bias)


def test_activation_applies_after_beta_and_bias():
    """relu(1*1 + 1*(-3) + 1.5) = relu(-0.5) = 0; the activation taken before
    the beta term would give 1 - 3 + 1.5, before the bias -2 + 1.5."""
    one = np.float32([[1.0]])
    out = oracle.gemm_epilogue_ref(one, one, 1.0, 1.0, np.float32([[-3.0]]), np.float32([1.5]), "relu")
    assert out[0, 0] == 0.0
    out = oracle.gemm_epilogue_ref(one, one, 1.0, 1.0, np.float32([[-3.0]]), np.float32([2.5]), "relu")
    assert out[0, 0] == 0.5


# ----------------------------------------------------------------------------- acceptance measure

def test_error_ratio_measure():
    ref = np.array([[1.0, 0.0, -2.0]])
    D = np.array([[2.0, 0.0, 4.0]])
    assert oracle.error_ratio(np.array([[1.0, 0.0, -2.0]]), ref, D) == 0.0
    assert oracle.error_ratio(np.array([[1.5, 0.0, -2.0]]), ref, D) == 0.25
    assert oracle.error_ratio(np.array([[1.0, 1e-30, -2.0]]), ref, D) == float("inf")
    assert oracle.error_ratio(np.array([[np.nan, 0.0, -2.0]]), ref, D) == float("inf")


def test_oracle_uses_threads():
    assert oracle.num_threads() >= 1


# ----------------------------------------------------------------------------- output quantisation

def _e4m3_values():
    """The 127 non-negative finite E4M3 values in code order, decoded by the
    format's definition (exponent bias 7, subnormals m * 2^-9)."""
    vals = []
    for c in range(127):
        e, m = (c >> 3) & 15, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_quantize_e4m3_round_trips_every_finite_code():
    v = _e4m3_values()
    assert v[-1] == 448.0 and np.all(np.diff(v) > 0)
    both = np.concatenate([v, -v])
    np.testing.assert_array_equal(oracle.quantize(both, "fp8"), both)


def test_quantize_e4m3_ties_go_to_the_even_code():
    v = _e4m3_values()
    mid = (v[:-1] + v[1:]) / 2          # exact in fp64
    even = np.where(np.arange(126) % 2 == 0, v[:-1], v[1:])
    np.testing.assert_array_equal(oracle.quantize(mid, "fp8"), even)
    np.testing.assert_array_equal(oracle.quantize(-mid, "fp8"), -even)
    gap = v[1:] - v[:-1]
    np.testing.assert_array_equal(oracle.quantize(mid - gap / 8, "fp8"), v[:-1])
    np.testing.assert_array_equal(oracle.quantize(mid + gap / 8, "fp8"), v[1:])


def test_quantize_e4m3_saturates_and_keeps_nan_and_signed_zero():
    x = np.array([448.0, 449.0, 463.99, 464.0, 1e30, np.inf, -500.0, -np.inf])
    np.testing.assert_array_equal(oracle.quantize(x, "fp8"), [448, 448, 448, 448, 448, 448, -448, -448])
    q = oracle.quantize(np.array([np.nan, -0.0, 0.0]), "fp8")
    assert np.isnan(q[0]) and np.signbit(q[1]) and not np.signbit(q[2])


def test_quantize_e4m3_matches_torch_in_range():
    """torch's own E4M3 conversion (round to nearest even) on fp32 values
    below 464, past which torch gives NaN where the oracle saturates."""
    rng = np.random.default_rng(41)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) < 464]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.quantize(x.astype(np.float64), "fp8"), t)


def test_quantize_bf16_matches_torch():
    """torch's fp32 -> bfloat16 conversion (round to nearest even) on random
    fp32 values, exact ties, subnormals and values near the top of the range."""
    rng = np.random.default_rng(42)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-38, 1e-3, 1.0, 1e20, 1e37)]).astype(np.float32)
    base = rng.standard_normal(5000).astype(np.float32)
    base = torch.from_numpy(base).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)     # exactly half a bf16 step up
    top = np.array([3.3895e38, 3.39e38, 3.3961e38, 3.4e38, np.finfo(np.float32).max], np.float32)
    x = np.concatenate([x, ties, -ties, top, -top])
    t = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(oracle.quantize(x.astype(np.float64), "bf16"), t)
    q = oracle.quantize(np.array([np.nan, -0.0]), "bf16")
    assert np.isnan(q[0]) and np.signbit(q[1])


def test_quantize_applies_the_scale_first():
    rng = np.random.default_rng(43)
    x = rng.standard_normal(1000) * 10
    for kind in ("bf16", "fp8"):
        np.testing.assert_array_equal(oracle.quantize(x, kind, scale=0.375), oracle.quantize(x * 0.375, kind))
