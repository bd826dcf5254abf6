"""The oracle's pins must catch plausible mistakes.

Each mutant below is the oracle source with one planted mistake (a dropped
term, a flipped sign, a wrong index, a transposed operand, an ignored leading
dimension, a wrong bf16 widening).  It is compiled on the CPU into a
temporary library and the whole pin suite (tests/test_oracle.py) is run
against it in a subprocess; the suite must fail for every mutant.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gemm_ref.c")

# (name, [(old, new, occurrence)])  -- occurrence counts matches of `old` in the source
MUTANTS = [
    ("beta_term_dropped", [("v += beta * (double)C0[i * ldc0 + j];", "(void)0;", 0)]),
    ("beta_sign_flipped", [("v += beta * (double)C0[i * ldc0 + j];", "v -= beta * (double)C0[i * ldc0 + j];", 0)]),
    ("alpha_dropped", [("double v = alpha * row[j];", "double v = row[j];", 0)]),
    ("B_transposed", [("const float *brow = B + k * ldb;", "const float *brow = B + k;", 0),
                      ("row[j] += a * (double)brow[j];", "row[j] += a * (double)brow[j * ldb];", 0)]),
    ("A_transposed", [("const double a = (double)A[i * lda + k];", "const double a = (double)A[k * lda + i];", 0)]),
    ("last_k_dropped", [("for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];",
                         "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a = (double)A[i * lda + k];", 0)]),
    ("first_k_dropped", [("for (int64_t k = 0; k < K; ++k) {\n            const double a = (double)A[i * lda + k];",
                          "for (int64_t k = 1; k < K; ++k) {\n            const double a = (double)A[i * lda + k];", 0)]),
    ("last_column_dropped", [("for (int64_t j = 0; j < N; ++j)\n                row[j] += a * (double)brow[j];",
                              "for (int64_t j = 0; j < N - 1; ++j)\n                row[j] += a * (double)brow[j];", 0)]),
    ("lda_ignored", [("A[i * lda + k]", "A[i * K + k]", 0)]),
    ("ldb_ignored", [("B + k * ldb;", "B + k * N;", 0)]),
    ("ldc_ignored", [("C0[i * ldc0 + j]", "C0[i * N + j]", 0)]),
    ("accumulator_not_cleared", [("row[j] = 0.0;", "row[j] = 1e-300 * (double)j;", 0)]),
    ("product_replaced_by_sum", [("row[j] += a * (double)brow[j];", "row[j] += a + (double)brow[j];", 0)]),
    ("term_subtracted", [("row[j] += a * (double)brow[j];", "row[j] -= a * (double)brow[j];", 0)]),
    ("bf16_wrong_shift", [("<< 16", "<< 15", 0)]),
    ("bf16_B_transposed", [("const uint16_t *brow = B + k * ldb;", "const uint16_t *brow = B + k;", 0),
                           ("row[j] += a * widen_bf16(brow[j]);", "row[j] += a * widen_bf16(brow[j * ldb]);", 0)]),
    ("bf16_beta_dropped", [("v += beta * (double)C0[i * ldc0 + j];", "(void)0;", 1)]),
    ("absbound_abs_of_B_dropped", [("row[j] += a * fabs((double)brow[j]);", "row[j] += a * (double)brow[j];", 0)]),
    ("absbound_beta_dropped", [("v += ab * fabs((double)C0[i * ldc0 + j]);", "(void)ab;", 0)]),
    ("absbound_alpha_signed", [("double v = aa * row[j];", "double v = alpha * row[j];", 0)]),
    ("epilogue_bias_dropped", [("z += (double)bias[j];", "(void)bias;", 0)]),
    ("epilogue_bias_row_index", [("z += (double)bias[j];", "z += (double)bias[i % N];", 0)]),
    ("epilogue_bias_after_activation", [("z += (double)bias[j];", "(void)0;", 0),
                                        ("Z[i * ldz + j] = z;", "Z[i * ldz + j] = z + (bias ? (double)bias[j] : 0.0);",
                                         0)]),
    ("relu_inverted", [("if (z < 0.0)", "if (z > 0.0)", 0)]),
    ("gelu_sqrt2_dropped", [("erf(z * inv_sqrt2)", "erf(z)", 0)]),
    ("gelu_half_dropped", [("z = 0.5 * z * (1.0 + erf", "z = z * (1.0 + erf", 0)]),
    ("gelu_erf_sign", [("(1.0 + erf(", "(1.0 - erf(", 0)]),
    ("e4m3_bias_wrong", [("v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 9);", 0)]),
    ("e4m3_subnormal_scale", [("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);", 0)]),
    ("e4m3_nan_missing", [("if (e == 15 && m == 7)\n        v = NAN;", "if (0)\n        v = NAN;", 0)]),
    ("e4m3_sign_ignored", [("return (bits & 0x80) ? -v : v;", "return v;", 0)]),
    ("fp8_beta_dropped", [("v += beta * (double)C0[i * ldc0 + j];", "(void)0;", 2)]),
    ("fp8_B_row_stride_ignored", [("const uint8_t *brow = B + k * ldb;", "const uint8_t *brow = B + k * N;", 0)]),
    ("groupmax_run_of_7", [("if (k % 8 == 7 || k == K - 1)", "if (k % 7 == 6 || k == K - 1)", 0)]),
    ("groupmax_sum_not_max", [("if (p > run[j])\n                    run[j] = p;", "run[j] += p;", 0)]),
    ("quant_e4m3_ties_up", [("r = (c % 2 == 0) ? lo : hi;", "r = hi;", 0)]),
    ("quant_e4m3_no_saturation", [("if (a >= 448.0) {\n        r = 448.0;", "if (a >= 448.0) {\n        r = a;", 0)]),
    ("quant_e4m3_truncates", [("if (a - lo < hi - a)\n            r = lo;", "if (1)\n            r = lo;", 0)]),
    ("quant_bf16_ties_up", [("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0))", "if (frac >= 0.5)", 0)]),
    ("quant_bf16_7_bits", [("int q = e - 8;", "int q = e - 7;", 0)]),
    ("quant_bf16_no_subnormals", [("q = -133;", "q = -126;", 0)]),
    ("quant_scale_dropped", [("const double v = scale * Z[i * ldz + j];", "const double v = Z[i * ldz + j];", 0)]),
]


def _apply(src: str, edits):
    for old, new, occ in edits:
        pos = -1
        for _ in range(occ + 1):
            pos = src.find(old, pos + 1)
            if pos < 0:
                raise AssertionError(f"mutation anchor not found: {old!r} (occurrence {occ})")
        src = src[:pos] + new + src[pos + len(old):]
    return src


def _run_mutant(name, edits, workdir):
    with open(SRC) as f:
        src = _apply(f.read(), edits)
    c_path = os.path.join(workdir, f"{name}.c")
    so_path = os.path.join(workdir, f"lib_{name}.so")
    with open(c_path, "w") as f:
        f.write(src)
    cmd = oracle.build_cmd(so_path, c_path)
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, GEMM_ORACLE_LIB=so_path, OMP_NUM_THREADS="2")
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
         "-x", "-q", "-p", "no:cacheprovider"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, proc.returncode, proc.stdout[-400:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_every_mutant_is_caught():
    workdir = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        # Control: the unmodified source through the same pipeline must pass.
        _, rc, out = _run_mutant("control", [], workdir)
        assert rc == 0, f"unmutated oracle fails its pins through the mutant harness: {out}"
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_mutant(m[0], m[1], workdir), MUTANTS))
    finally:
        shutil.rmtree(workdir, ignore_errors=True)
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants not caught by the oracle pins: {survivors}"
    # pytest exit 1 = tests failed; a negative code = the mutant crashed the
    # process.  Anything else (usage error, collection error) proves nothing.
    odd = [(n, rc, out) for n, rc, out in results if rc != 1 and rc >= 0]
    assert not odd, f"mutant runs ended for a reason other than a failed pin: {odd}"
