"""Seeded synthetic GEMM inputs shared by the tests, the smoke check and the
benchmark.

This module only draws random numbers; it holds none of the GEMM arithmetic.
Both the HIP library and the CPU oracle consume the same host arrays it
returns, so the generator's own rounding cannot break parity.

Recipe (fixed, so that every run sees the same bytes):

* ``g = torch.Generator('cpu').manual_seed(seed)`` for each workload.
* Draw order A, then B, then C0.  C0 is always drawn, even when ``beta == 0``,
  so the sequence does not depend on beta.
* ``uniform``: ``torch.empty(shape).uniform_(-1, 1, generator=g)``.
* ``normal``: ``torch.randn(shape, generator=g)``.
* bf16 operands: the fp32 draw rounded to bf16 with ``.to(torch.bfloat16)``
  (round to nearest even); C0 stays fp32.  fp8 operands likewise with
  ``.to(torch.float8_e4m3fn)`` (OCP E4M3, round to nearest even).
* A transposed operand (``op_a`` or ``op_b == "T"``) is drawn in its
  defining shape (M x K or K x N) and then stored transposed.

The shapes are the square and ragged problems the pages measure on (4092 and
4096 cubes on page 1 and page 3), a small cube, a ragged shape that is a
multiple of no tile size, a decode-like M = 16 shape (the bandwidth-bound
case the second page warns about) and a large bf16 cube.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32", "bf16f32" or "fp8f32" (bf16 / fp8 E4M3 operands, fp32 accumulate and output)
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str           # "uniform" (U[-1, 1]) or "normal" (N(0, 1))
    seed: int
    op_b: str = "N"     # "T": B is stored transposed (N x K)
    op_a: str = "N"     # "T": A is stored transposed (K x M)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elt_bytes(self) -> int:
        return {"f32": 4, "bf16f32": 2, "fp8f32": 1}[self.dtype]

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the operation must move: read A and B (and C0 if beta != 0), write C."""
        ab = (self.M * self.K + self.K * self.N) * self.elt_bytes
        c = self.M * self.N * 4
        return ab + c * (2 if self.beta != 0.0 else 1)


WORKLOADS = {
    w.name: w for w in [
        Workload("f32_256", "f32", 256, 256, 256, 1.0, 0.0, "uniform", 0),
        Workload("f32_4092_beta", "f32", 4092, 4092, 4092, 1.0, 0.5, "uniform", 1),
        Workload("f32_4096", "f32", 4096, 4096, 4096, 1.0, 0.0, "normal", 2),
        Workload("f32_1000x3000x777", "f32", 1000, 3000, 777, 2.0, -1.0, "uniform", 3),
        Workload("f32_16x8192x8192", "f32", 16, 8192, 8192, 1.0, 0.0, "uniform", 3),
        Workload("bf16f32_8192", "bf16f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 4),
        # fp8 operands with B stored N x K, the layout of the fp8 matrix-core kernel.
        Workload("fp8f32_8192_nt", "fp8f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 5, "T"),
        Workload("bf16f32_8192_nt", "bf16f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 6, "T"),
        Workload("bf16f32_8192_tn", "bf16f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 7, "N", "T"),
        Workload("bf16f32_16x8192x8192", "bf16f32", 16, 8192, 8192, 1.0, 0.0, "normal", 8),
        Workload("bf16f32_16x8192x8192_nt", "bf16f32", 16, 8192, 8192, 1.0, 0.0, "normal", 9, "T"),
        Workload("f32_16x8192x8192_nt", "f32", 16, 8192, 8192, 1.0, 0.0, "uniform", 10, "T"),
        Workload("fp8f32_16x8192x8192_nt", "fp8f32", 16, 8192, 8192, 1.0, 0.0, "normal", 11, "T"),
        Workload("f32_4096_nt", "f32", 4096, 4096, 4096, 1.0, 0.0, "normal", 12, "T"),
        Workload("f32_4096_tn", "f32", 4096, 4096, 4096, 1.0, 0.0, "normal", 13, "N", "T"),
        Workload("fp8f32_8192_nn", "fp8f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 14),
        Workload("fp8f32_8192_tn", "fp8f32", 8192, 8192, 8192, 1.0, 0.0, "normal", 15, "N", "T"),
        # Mid-size: 512 tiles of 128^2 (two workgroups per compute unit), 128 of 256^2.
        Workload("bf16f32_2048x4096x4096", "bf16f32", 2048, 4096, 4096, 1.0, 0.0, "normal", 16),
        Workload("bf16f32_2048x4096x4096_nt", "bf16f32", 2048, 4096, 4096, 1.0, 0.0, "normal", 17, "T"),
        Workload("f32_2048x4096x4096", "f32", 2048, 4096, 4096, 1.0, 0.0, "normal", 18),
    ]
}


def _draw(shape, dist: str, g: torch.Generator) -> torch.Tensor:
    if dist == "uniform":
        return torch.empty(shape, dtype=torch.float32).uniform_(-1.0, 1.0, generator=g)
    if dist == "normal":
        return torch.randn(shape, dtype=torch.float32, generator=g)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload):
    """Host tensors (A, B, C0) for a workload.

    A and B are float32 for ``f32`` workloads, bfloat16 for ``bf16f32`` and
    float8_e4m3fn for ``fp8f32``; B is returned as stored (N x K when
    ``op_b == "T"``).  C0 is always float32 of shape (M, N).
    """
    g = torch.Generator("cpu").manual_seed(w.seed)
    A = _draw((w.M, w.K), w.dist, g)
    B = _draw((w.K, w.N), w.dist, g)
    C0 = _draw((w.M, w.N), w.dist, g)
    A, B = _operand_type(A, w.dtype), _operand_type(B, w.dtype)
    if w.op_b == "T":
        B = B.t().contiguous()
    if w.op_a == "T":
        A = A.t().contiguous()
    return A, B, C0


def _operand_type(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """fp32 draws rounded (nearest even) to the operand type: "f32", "bf16f32"
    or "fp8f32" (OCP E4M3; N(0,1) and small-integer draws stay far inside its
    finite range)."""
    if dtype == "bf16f32":
        return x.to(torch.bfloat16)
    if dtype == "fp8f32":
        return x.to(torch.float8_e4m3fn)
    assert dtype == "f32", dtype
    return x


def make_integer_inputs(M: int, N: int, K: int, seed: int, lo: int = -4, hi: int = 4,
                        dtype: str = "f32"):
    """Small-integer operands (exact in fp32, bf16 and fp8 E4M3) and an integer C0.

    With |entries| <= 4 every partial sum stays an integer below 2**24 for
    K < 2**20, so any summation order gives the same exact result.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    A = torch.randint(lo, hi + 1, (M, K), generator=g).to(torch.float32)
    B = torch.randint(lo, hi + 1, (K, N), generator=g).to(torch.float32)
    C0 = torch.randint(lo, hi + 1, (M, N), generator=g).to(torch.float32)
    return _operand_type(A, dtype), _operand_type(B, dtype), C0


def make_bias(N: int, seed: int, dist: str = "normal", integer: bool = False):
    """A float32 bias vector of N values (seeded; small integers if asked)."""
    g = torch.Generator("cpu").manual_seed(seed)
    if integer:
        return torch.randint(-4, 5, (N,), generator=g).to(torch.float32)
    return _draw((N,), dist, g)


def make_random_inputs(M: int, N: int, K: int, seed: int, dist: str = "uniform",
                       dtype: str = "f32"):
    """Random operands of an arbitrary shape with the same draw order."""
    g = torch.Generator("cpu").manual_seed(seed)
    A = _draw((M, K), dist, g)
    B = _draw((K, N), dist, g)
    C0 = _draw((M, N), dist, g)
    return _operand_type(A, dtype), _operand_type(B, dtype), C0


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bfloat16 tensor's bit patterns (for the oracle)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def fp8_bytes(t: torch.Tensor):
    """uint8 numpy view of a float8_e4m3fn tensor's bytes (for the oracle)."""
    assert t.dtype == torch.float8_e4m3fn
    return t.contiguous().view(torch.uint8).numpy()
