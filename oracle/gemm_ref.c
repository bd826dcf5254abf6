/*
 * Reference GEMM oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, deliberately obvious CPU implementation of the operation the
 * pages define:
 *
 *     C = alpha * (A x B) + beta * C0,   A is M x K, B is K x N, C is M x N
 *
 * ("GEMM Worklog I: Naive to Tiled", opening formula; "A GEMM Kernel, Step by
 * Step", section "The ladder we are climbing", which states the problem as
 * one call C <- alpha*A*B + beta*C).  Entry (i, j) is the dot product of row
 * i of A with column j of B, exactly as the naive kernel of the first page
 * computes it (section 1, "The Naive CUDA Kernel"), scaled by alpha, plus
 * beta times the old entry.
 *
 * Precision: every input element is widened exactly to double (fp32 -> fp64
 * is exact; a bf16 bit pattern shifted left by 16 is an exact fp32 value,
 * hence exact in fp64).  Each product of two such values is exact in fp64
 * (24 + 24 significand bits <= 53), so the only rounding is the fp64
 * accumulation over k, which runs in ascending k for every entry.
 *
 * Loop order: the i-k-j nest below adds the terms of each entry C[i][j] in
 * the same order (k = 0, 1, ..., K-1) as the textbook i-j-k dot product;
 * only the traversal of independent entries differs, so the result is
 * bitwise the same as the triple loop.  Rows are independent and are spread
 * over OpenMP threads; nothing is blocked, fused or reordered within an
 * entry.
 *
 * Conventions where the pages are silent (each is listed in the design
 * notes): row-major storage with explicit leading dimensions
 * (A[i*lda+k], B[k*ldb+j], C[i*ldc+j]); when beta == 0 the beta*C0 term is
 * omitted entirely, so C0 is never read and NaN/Inf in it cannot propagate;
 * K == 0 gives an empty sum (0).
 *
 * This library shares no code, header or constant with the HIP path.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* out[i*ldo + j] = alpha * sum_k A[i][k] * B[k][j]  (+ beta * C0[i][j] when beta != 0) */
void gemm_ref_f32in(int64_t M, int64_t N, int64_t K, double alpha,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double beta, const float *C0, int64_t ldc0,
                    double *out, int64_t ldo)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * (double)brow[j];
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * row[j];
            if (beta != 0.0)
                v += beta * (double)C0[i * ldc0 + j];
            row[j] = v;
        }
    }
}

/* Same definition with bf16 operands (raw bit patterns), fp32 C0. */
void gemm_ref_bf16in(int64_t M, int64_t N, int64_t K, double alpha,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                     double beta, const float *C0, int64_t ldc0,
                     double *out, int64_t ldo)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = widen_bf16(A[i * lda + k]);
            const uint16_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * widen_bf16(brow[j]);
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * row[j];
            if (beta != 0.0)
                v += beta * (double)C0[i * ldc0 + j];
            row[j] = v;
        }
    }
}

/*
 * Error-bound denominator for the acceptance test:
 *     D[i][j] = |alpha| * sum_k |A[i][k]| * |B[k][j]|  (+ |beta| * |C0[i][j]| when beta != 0)
 * A floating-point evaluation of the GEMM in any summation order has error
 * bounded by a small multiple of the unit roundoff times this sum (standard
 * forward error bound of an inner product), so |C_gpu - C_ref| / D is the
 * scale-free error measure.
 */
void gemm_absbound_f32in(int64_t M, int64_t N, int64_t K, double alpha,
                         const float *A, int64_t lda, const float *B, int64_t ldb,
                         double beta, const float *C0, int64_t ldc0,
                         double *out, int64_t ldo)
{
    const double aa = fabs(alpha);
    const double ab = fabs(beta);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = fabs((double)A[i * lda + k]);
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * fabs((double)brow[j]);
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = aa * row[j];
            if (beta != 0.0)
                v += ab * fabs((double)C0[i * ldc0 + j]);
            row[j] = v;
        }
    }
}

void gemm_absbound_bf16in(int64_t M, int64_t N, int64_t K, double alpha,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          double beta, const float *C0, int64_t ldc0,
                          double *out, int64_t ldo)
{
    const double aa = fabs(alpha);
    const double ab = fabs(beta);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = fabs(widen_bf16(A[i * lda + k]));
            const uint16_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * fabs(widen_bf16(brow[j]));
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = aa * row[j];
            if (beta != 0.0)
                v += ab * fabs((double)C0[i * ldc0 + j]);
            row[j] = v;
        }
    }
}

/*
 * fp8 operands: the OCP 8-bit floating-point format E4M3 (the variant with
 * no infinities), raw bytes.  Bit 7 is the sign, bits 6..3 the exponent with
 * bias 7, bits 2..0 the mantissa.  Exponent field 0 is subnormal, m * 2^-9;
 * exponent 15 with mantissa 7 is NaN; every other code is finite (the
 * largest is 448).  Every value is exact in double, and so is every product
 * of two of them.
 */
static double widen_e4m3(uint8_t bits)
{
    const int e = (bits >> 3) & 15, m = bits & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10);          /* (1 + m/8) * 2^(e-7) */
    return (bits & 0x80) ? -v : v;
}

/* The GEMM definition with fp8 E4M3 operands (raw bytes), fp32 C0. */
void gemm_ref_fp8in(int64_t M, int64_t N, int64_t K, double alpha,
                    const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                    double beta, const float *C0, int64_t ldc0,
                    double *out, int64_t ldo)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = widen_e4m3(A[i * lda + k]);
            const uint8_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * widen_e4m3(brow[j]);
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = alpha * row[j];
            if (beta != 0.0)
                v += beta * (double)C0[i * ldc0 + j];
            row[j] = v;
        }
    }
}

/* The error-ratio denominator (as above) with fp8 operands. */
void gemm_absbound_fp8in(int64_t M, int64_t N, int64_t K, double alpha,
                         const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         double beta, const float *C0, int64_t ldc0,
                         double *out, int64_t ldo)
{
    const double aa = fabs(alpha);
    const double ab = fabs(beta);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        for (int64_t j = 0; j < N; ++j)
            row[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = fabs(widen_e4m3(A[i * lda + k]));
            const uint8_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j)
                row[j] += a * fabs(widen_e4m3(brow[j]));
        }
        for (int64_t j = 0; j < N; ++j) {
            double v = aa * row[j];
            if (beta != 0.0)
                v += ab * fabs((double)C0[i * ldc0 + j]);
            row[j] = v;
        }
    }
}

/*
 * Group-maximum bound for fp8 products summed in runs of 8:
 *     G[i][j] = |alpha| * sum over q of max_{8q <= k < min(8q+8, K)} |A[i][k] * B[k][j]|
 * A sum that aligns each run of 8 consecutive products to the run's largest
 * and keeps a fixed number of bits below it loses less than one unit of the
 * last kept bit per product; this sum of run maxima scales that loss.
 */
void gemm_groupmax_fp8in(int64_t M, int64_t N, int64_t K, double alpha,
                         const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         double *out, int64_t ldo)
{
    const double aa = fabs(alpha);
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *row = out + i * ldo;
        double *run = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        for (int64_t j = 0; j < N; ++j) {
            row[j] = 0.0;
            run[j] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double a = fabs(widen_e4m3(A[i * lda + k]));
            const uint8_t *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                const double p = a * fabs(widen_e4m3(brow[j]));
                if (p > run[j])
                    run[j] = p;
            }
            if (k % 8 == 7 || k == K - 1) {
                for (int64_t j = 0; j < N; ++j) {
                    row[j] += run[j];
                    run[j] = 0.0;
                }
            }
        }
        for (int64_t j = 0; j < N; ++j)
            row[j] *= aa;
        free(run);
    }
}

/*
 * Fused epilogue, applied to a finished GEMM result Z (M x N, fp64, row
 * stride ldz) in place:
 *
 *     Z[i][j] <- act(Z[i][j] + bias[j])
 *
 * ("Tiled matrix multiplication", sections "Efficiency" and "Implementation
 * notes": bias and activation are applied to the GEMM result while it is
 * still in registers.)  The pages name the operations but define neither
 * activation; the readings taken are the usual ones:
 *   act == 0  identity;
 *   act == 1  ReLU, max(z, 0); a NaN compares false and is kept;
 *   act == 2  GELU, z * Phi(z) with Phi the standard normal CDF, written
 *             through the error function: Phi(z) = (1 + erf(z / sqrt 2)) / 2,
 *             using the C library's double erf.
 * bias is NULL (no bias) or N floats, widened exactly to double.
 */
void epilogue_ref(int64_t M, int64_t N, double *Z, int64_t ldz, const float *bias, int act)
{
    const double inv_sqrt2 = 1.0 / sqrt(2.0);
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double z = Z[i * ldz + j];
            if (bias != NULL)
                z += (double)bias[j];
            if (act == 1) {
                if (z < 0.0)
                    z = 0.0;
            } else if (act == 2) {
                z = 0.5 * z * (1.0 + erf(z * inv_sqrt2));
            }
            Z[i * ldz + j] = z;
        }
    }
}

/*
 * Output quantisation, the last fused epilogue step ("Tiled matrix
 * multiplication", sections "Efficiency" and "Implementation notes": the
 * result is converted while still in registers, before it is stored).  The
 * pages name the step but fix no format or rounding; the readings taken:
 * the value is multiplied by `scale`, then rounded to the nearest value of
 * the storage format, ties to the even code (IEEE round-to-nearest-even).
 *
 *   kind 1: bfloat16, 8 significant bits over fp32's exponent range
 *           (normal down to 2^-126, subnormal steps of 2^-133).  Past the
 *           largest finite value the rounding reaches infinity, as IEEE
 *           rounding does.
 *   kind 2: OCP E4M3 (see widen_e4m3).  The format has no infinities:
 *           magnitudes at or past the largest finite value, 448, give +-448
 *           (saturation).
 *
 * NaN stays NaN; the sign of zero is kept.
 */
static double quant_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    const double a = fabs(x);
    int e;
    frexp(a, &e);                          /* a = f * 2^e, 0.5 <= f < 1 */
    int q = e - 8;                         /* spacing of 8-bit significands in this binade */
    if (q < -133)
        q = -133;                          /* subnormal spacing */
    const double ulp = ldexp(1.0, q);
    const double n = a / ulp;              /* exact: ulp is a power of two */
    const double fl = floor(n), frac = n - fl;
    double m = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0))
        m = fl + 1.0;
    double r = m * ulp;
    const double max_finite = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (r > max_finite)
        r = INFINITY;
    return copysign(r, x);
}

static double quant_e4m3(double x)
{
    if (isnan(x))
        return x;
    const double a = fabs(x);
    double r;
    if (a >= 448.0) {
        r = 448.0;
    } else {
        /* Codes 0 .. 126 are the non-negative finite values in increasing
         * order; find the two that bracket a. */
        int c = 0;
        while (c < 126 && widen_e4m3((uint8_t)(c + 1)) <= a)
            ++c;
        const double lo = widen_e4m3((uint8_t)c), hi = widen_e4m3((uint8_t)(c + 1));
        if (a - lo < hi - a)
            r = lo;
        else if (a - lo > hi - a)
            r = hi;
        else
            r = (c % 2 == 0) ? lo : hi;
    }
    return copysign(r, x);
}

/* Z[i][j] <- quantise(scale * Z[i][j]) for kind 1 (bf16) or 2 (E4M3). */
void quantize_ref(int64_t M, int64_t N, double *Z, int64_t ldz, int kind, double scale)
{
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            const double v = scale * Z[i * ldz + j];
            Z[i * ldz + j] = kind == 1 ? quant_bf16(v) : quant_e4m3(v);
        }
    }
}

/* Threads OpenMP will use for the loops above (reported next to timings). */
int gemm_ref_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
