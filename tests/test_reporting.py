"""Pins for the cost-model helpers against numbers the pages print.

Each case in tests/golden/*.json names the page and section it comes from.
"""
import json
import os

import pytest

from tiled_gemm_f32_amd import roofline as rl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_intensity_table_reprints_page_values():
    t = _load("intensity_table.json")
    peak, bw = t["peak_flops"], t["bandwidth"]
    for row in t["rows"]:
        i = rl.tile_intensity(row["m"], row["n"], 4)
        assert round(i, 2) == pytest.approx(row["flop_per_byte"], abs=1e-9), row
        assert round(rl.roofline_ceiling(i, peak, bw) / 1e9) == row["ceiling_gflops"], row
    assert round(rl.ridge_point(peak, bw), 2) == pytest.approx(t["ridge_flop_per_byte"])


def _evaluate(kind, args):
    if kind == "gemm_flops":
        return rl.gemm_flops(*args)
    if kind == "naive_bytes":          # two 4-byte loads for every multiply-add
        M, N, K = args
        return M * N * K * 2 * 4
    if kind == "tile_intensity":
        return rl.tile_intensity(*args)
    if kind == "ridge":
        return rl.ridge_point(*args)
    if kind == "ceiling":
        return rl.roofline_ceiling(*args)
    if kind == "ratio":
        return args[0] / args[1]
    if kind == "rate":
        M, N, K, t = args
        return rl.gemm_flops(M, N, K) / t
    if kind == "floor_read":
        n = args[0]
        return rl.memory_floor_bytes(n, n, n, 4, read_c=True) - n * n * 4
    if kind == "floor_write":
        n = args[0]
        return n * n * 4
    if kind == "memory_floor":
        return rl.memory_floor_bytes(*args, 4, read_c=True)
    if kind == "problem_intensity":
        n = args[0]
        return rl.gemm_flops(n, n, n) / rl.memory_floor_bytes(n, n, n, 4, read_c=True)
    if kind == "seconds":
        return args[0] / args[1]
    if kind == "tiles_per_side":
        return rl.tiles_per_side(*args)
    if kind == "overhang":
        return 1.0 / rl.tile_quantisation(*args) - 1.0
    if kind == "tile_quantisation":
        return rl.tile_quantisation(*args)
    if kind == "wave_count":
        return rl.wave_count(*args)
    if kind == "wave_efficiency":
        return rl.wave_efficiency(*args)
    if kind == "bf16_operands":       # A, B and C of an n-cube at 2 bytes each
        n = args[0]
        return rl.memory_floor_bytes(n, n, n, 2, read_c=False, c_bytes=2)
    if kind == "smem_bytes":          # transposed A panel [BK][BM+pad] plus B panel [BK][BN], fp32
        BM, BN, BK, pad = args
        return (BK * (BM + pad) + BK * BN) * 4
    raise KeyError(kind)


CASES = _load("worked_numbers.json")["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_worked_numbers(case):
    got = _evaluate(case["kind"], case["args"])
    want = case["printed"]
    if case["rel_tol"] == 0:
        assert got == pytest.approx(want, rel=1e-12, abs=1e-12), case["cite"]
    else:
        assert abs(got - want) <= case["rel_tol"] * abs(want), (got, case["cite"])


def test_mi355x_peaks_follow_unit_counts():
    """fp32 matrix peak = 256 FLOP/CU/clk, bf16 = 4096 FLOP/CU/clk at 2.4 GHz x 256 CUs."""
    base = rl.MI355X_CUS * rl.MI355X_CLOCK_HZ
    assert base * 256 == pytest.approx(rl.MI355X_FP32_MATRIX_FLOPS, rel=1e-3)
    assert base * 4096 == pytest.approx(2516.6e12, rel=1e-4)
    assert rl.MI355X_BF16_MATRIX_FLOPS == pytest.approx(base * 4096, rel=0.01)
