"""Cost-model helpers used when reporting GEMM throughput.

These follow the cost analysis of "A GEMM Kernel, Step by Step" (section
"What the problem is allowed to cost"): the arithmetic is fixed at 2MNK
floating-point operations, the memory floor is one read of every operand and
one write of the result, and a block tile of shape m x n fed from DRAM runs at
an arithmetic intensity of m*n / (2*(m + n)) FLOP per byte for 4-byte
elements (each k step moves m + n elements and performs 2*m*n operations).
The roofline ceiling of a kernel at intensity I is min(peak, I * bandwidth).

The MI355X figures are the published dense peaks at the 2.4 GHz engine clock.
"""
from __future__ import annotations

import math

# Published MI355X peaks (dense, no sparsity).
MI355X_CUS = 256
MI355X_CLOCK_HZ = 2.4e9
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_FP32_MATRIX_FLOPS = 157.3e12
MI355X_BF16_MATRIX_FLOPS = 2.5e15       # 2516.6 TFLOP/s computed from 4096 FLOP/CU/clk
MI355X_FP32_VECTOR_FLOPS = 157.3e12
MI355X_FP64_VECTOR_FLOPS = 78.6e12


def gemm_flops(M: int, N: int, K: int) -> int:
    """Operation count of C = alpha*A*B + beta*C: 2*M*N*K (one multiply and one add per term)."""
    return 2 * M * N * K


def tile_intensity(m: int, n: int, elt_bytes: int = 4) -> float:
    """FLOP per byte of an m x n block tile whose operands stream from memory.

    Per step of k the tile reads m elements of A and n of B and performs 2*m*n
    operations, so I = 2*m*n / (elt_bytes*(m + n)); for 4-byte elements this is
    m*n / (2*(m + n)).
    """
    return 2.0 * m * n / (elt_bytes * (m + n))


def roofline_ceiling(intensity: float, peak_flops: float, bandwidth: float) -> float:
    """Attainable FLOP/s at a given intensity: min(peak, intensity * bandwidth)."""
    return min(peak_flops, intensity * bandwidth)


def ridge_point(peak_flops: float, bandwidth: float) -> float:
    """Intensity at which the memory slope meets the compute roof."""
    return peak_flops / bandwidth


def memory_floor_bytes(M: int, N: int, K: int, elt_bytes: int = 4,
                       read_c: bool = True, c_bytes: int = 4) -> int:
    """Minimum DRAM traffic: read A and B (and the old C), write the new C once."""
    return (M * K + K * N) * elt_bytes + M * N * c_bytes * (2 if read_c else 1)


def tiles_per_side(extent: int, tile: int) -> int:
    """Tiles of width ``tile`` needed to cover ``extent`` (the grid rounds up)."""
    return -(-extent // tile)


def tile_quantisation(M: int, N: int, BM: int, BN: int) -> float:
    """Fraction of the positions a tiled launch computes that lie inside C."""
    return (M * N) / (tiles_per_side(M, BM) * BM * tiles_per_side(N, BN) * BN)


def wave_count(tiles: int, slots: int) -> float:
    """Waves of a launch: tiles divided by the blocks the machine holds at once."""
    return tiles / slots


def wave_efficiency(tiles: int, slots: int) -> float:
    """Busy fraction when a launch of ``tiles`` equal blocks runs in whole waves."""
    return tiles / (math.ceil(tiles / slots) * slots)

