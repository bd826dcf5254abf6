/*
 * libgemm -- blocked general matrix multiply for AMD Instinct MI355X (gfx950).
 *
 *     C = alpha * (A x B) + beta * C
 *
 * with A of M x K, B of K x N and C of M x N, all row-major.  This is the
 * operation defined at the opening of "GEMM Worklog I: Naive to Tiled" and
 * posed as a single call in "A GEMM Kernel, Step by Step" (section "The
 * ladder we are climbing"); the host launcher shape (sizes, operand pointers,
 * a stream) follows the "Code" section of "Tiled matrix multiplication",
 * extended with alpha, beta and leading dimensions.
 *
 * Layout.  Element (i, k) of A is A[i*lda + k]; (k, j) of B is B[k*ldb + j];
 * (i, j) of C is C[i*ldc + j].  Requirements: lda >= max(1, K),
 * ldb >= max(1, N), ldc >= max(1, N).  Padding between rows is never read
 * in a way that can reach C (it may hold anything, NaN included).
 *
 * Memory.  A, B and C (and a workspace, where one is passed) are DEVICE
 * pointers on the current HIP device.  The caller owns them; the library
 * allocates nothing and keeps no state between calls ("Tiled matrix
 * multiplication", section "How it works": no state between calls).  C must
 * not overlap A or B.
 *
 * Streams.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL means the default stream) and the call returns without waiting.  The
 * result is visible after the stream is synchronised.  Calls on one stream
 * run in order.
 *
 * Scalars.  alpha and beta are fp32.  When beta == 0, C is write-only: its
 * old contents are never read, so NaN/Inf there does not propagate (the BLAS
 * convention; the pages leave this open).  When K == 0 or alpha == 0, A and
 * B are not read and C becomes beta * C (or 0).
 *
 * Errors.  Every function returns a gemm_status.  Argument checks happen
 * before any HIP call, so an invalid call has no side effect.
 * GEMM_ERR_LAUNCH reports a HIP error raised by the kernel launch (the
 * stream may then be unusable).  No function throws or aborts.
 */
#ifndef LIBGEMM_GEMM_H
#define LIBGEMM_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these entry points are exported. */
#define GEMM_API __attribute__((visibility("default")))

typedef enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,  /* negative size, leading dimension too small, NULL or
                                  misaligned pointer for an operand that is read or written */
    GEMM_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels index: M, N, K, lda or
                                  ldb above 2^31 - 1; or a forced kernel that cannot run on
                                  these operands */
    GEMM_ERR_LAUNCH = 3,       /* the HIP runtime reported an error for the launch */
    GEMM_ERR_DEVICE = 4,       /* no usable gfx950 device is current */
    GEMM_ERR_SCRATCH = 5       /* gemm_general_noalloc: the problem's K split could need more
                                  scratch than the library's static buffer holds */
} gemm_status;

/* A hipStream_t, passed through as an opaque pointer; NULL = default stream. */
typedef void *gemm_stream_t;

/*
 * fp32 GEMM.  Products and sums are fp32 (matrix-core fp32 multiply-add);
 * accumulation covers all of K before alpha and beta are applied.
 * M <= 16 takes the bandwidth-oriented skinny path (the decode-GEMV case of
 * "Tiled matrix multiplication", section "Avoid when"); every other shape
 * takes the LDS-tiled MFMA path.
 */
GEMM_API gemm_status gemm_f32(int64_t M, int64_t N, int64_t K, float alpha,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float beta, float *C, int64_t ldc,
                     gemm_stream_t stream);

/*
 * bf16 operands, fp32 accumulate and fp32 C.  A and B hold bfloat16 bit
 * patterns (uint16_t).  Each bf16 x bf16 product is exact in fp32; sums are
 * fp32.  The tensor-core variant of the blocked method ("Tiled matrix
 * multiplication", section "How it works", tensor-core level).
 */
GEMM_API gemm_status gemm_bf16f32(int64_t M, int64_t N, int64_t K, float alpha,
                         const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb,
                         float beta, float *C, int64_t ldc,
                         gemm_stream_t stream);

/*
 * Workspace.  These paths split K across workgroups and reduce the partial
 * results in a caller-provided device workspace (the split-K variant of
 * "Tiled matrix multiplication", section "Variants and alternatives", and of
 * "A GEMM Kernel, Step by Step", section "What is left"):
 *   - M <= 16 (fp32 and bf16; with B stored N x K through gemm_general, fp8
 *     too): the skinny streaming kernels, split into up to 8 k ranges of at
 *     least 512 while the strips of C (128 columns, or 32 with B stored
 *     N x K) number fewer than the 256 compute units;
 *   - any tiled problem with fewer output tiles than compute units: the
 *     tiled kernel, split into up to 16 k ranges of at least 1024, when the
 *     split grid fills at least three quarters of the compute units;
 *   - a tiled problem whose tile count is just over a multiple of the 256
 *     compute units (a last wave at most half full; "The fringe and the last
 *     wave", and the aim of Stream-K in "Variants and alternatives"): the
 *     top rows of tiles run first in whole waves, then the leftover bottom
 *     rows run K-split, spreading their work over the otherwise idle
 *     compute units (gemm_plan.split_row gives the boundary).
 * gemm_workspace_size() returns the largest workspace any path can use
 * for this shape (0 when none applies): `splits` partial fp32 results for
 * the rows split, reduced in split order by a further kernel on the same
 * stream (results are deterministic).  The workspace needs no initialisation and
 * its contents after a call are unspecified.  Calls sharing a workspace
 * must be ordered (same stream, or synchronised streams); overlapping calls
 * on one workspace race.  gemm_f32_ws() and gemm_bf16f32_ws() are
 * gemm_f32() and gemm_bf16f32() with a workspace; a NULL or too-small
 * workspace simply selects the workspace-free kernels.
 */
GEMM_API int64_t gemm_workspace_size(int32_t dtype, int64_t M, int64_t N, int64_t K);

GEMM_API gemm_status gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha,
                                 const float *A, int64_t lda, const float *B, int64_t ldb,
                                 float beta, float *C, int64_t ldc,
                                 void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

GEMM_API gemm_status gemm_bf16f32_ws(int64_t M, int64_t N, int64_t K, float alpha,
                                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                                    float beta, float *C, int64_t ldc,
                                    void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

/* Static English text for a status code (never NULL). */
GEMM_API const char *gemm_status_string(gemm_status status);

/* ------------------------------------------------------------------------
 * Kernel selection.  The library ships several kernels and picks one per
 * call from the shape, the alignment and the tile count against the 256
 * compute units ("A GEMM Kernel, Step by Step", section "Six parameters,
 * found by search": the library picks among kernels at run time by shape).
 * The functions below expose that choice so it can be inspected and tested.
 * ---------------------------------------------------------------------- */

typedef enum gemm_path {
    GEMM_PATH_NONE = 0,     /* quick return: nothing launched (M == 0 or N == 0) */
    GEMM_PATH_SCALE = 1,    /* C = beta * C only (K == 0 or alpha == 0) */
    GEMM_PATH_TILED = 2,    /* LDS-tiled MFMA kernel */
    GEMM_PATH_SKINNY = 3,   /* M <= 16 streaming kernel */
    GEMM_PATH_SKINNY_SPLITK = 4  /* M <= 16 streaming kernel with K split over workgroups
                                    (needs the caller's workspace) */
} gemm_path;

typedef enum gemm_dtype {
    GEMM_DTYPE_F32 = 0,     /* fp32 operands */
    GEMM_DTYPE_BF16F32 = 1, /* bf16 operands, fp32 accumulate and output */
    GEMM_DTYPE_FP8F32 = 2   /* fp8 operands (OCP E4M3, one byte each), fp32 accumulate and
                               output; gemm_general only */
} gemm_dtype;

/*
 * Operand layouts (gemm_general).  GEMM_OP_N: the operand is stored as
 * defined above (A: M x K, element (i, k) at A[i*lda + k]; B: K x N,
 * element (k, j) at B[k*ldb + j]).  GEMM_OP_T: it is stored transposed
 * (A: K x M, element (i, k) at A[k*lda + i], lda >= max(1, M); B: N x K,
 * element (k, j) at B[j*ldb + k], ldb >= max(1, K)).  The pages show the
 * untransposed layout only; the transposed ones are the usual weight
 * layouts (B as N x K).
 */
typedef enum gemm_op {
    GEMM_OP_N = 0,
    GEMM_OP_T = 1
} gemm_op;

typedef struct gemm_kernel_info {
    int32_t id;             /* 1-based; 0 is never a kernel */
    int32_t dtype;          /* gemm_dtype */
    int32_t path;           /* gemm_path (TILED, SKINNY or SKINNY_SPLITK) */
    int32_t tile_m, tile_n, tile_k;  /* workgroup tile (skinny: rows covered, columns, k unroll) */
    int32_t threads;        /* threads per workgroup */
    int32_t vec_a, vec_b;   /* elements per global load of A and of B (1 = element loads) */
    const char *name;       /* static string */
    int32_t layouts;        /* bit 2*op_a + op_b set for every operand layout it runs */
    int32_t outputs;        /* bit gemm_output set for every output type it writes */
} gemm_kernel_info;

typedef struct gemm_plan {
    int32_t path;           /* gemm_path */
    int32_t kernel_id;      /* kernel chosen (0 for NONE / SCALE) */
    int64_t grid;           /* workgroups launched (0 for NONE) */
    int32_t threads;        /* threads per workgroup */
    int32_t tile_m, tile_n, tile_k;
    int32_t vec_a, vec_b;
    int32_t splits;         /* k ranges of a tiled K split (1: none; 0 for NONE / SCALE) */
    int64_t split_row;      /* first row of C that the K split covers: rows above it run first,
                               unsplit, in whole waves of tiles (0: the split, if any, covers all) */
} gemm_plan;

/* Number of kernels in the table; ids run from 1 to this value. */
GEMM_API int32_t gemm_kernel_count(void);

/* Description of kernel `id`.  GEMM_ERR_INVALID_ARG for an unknown id or NULL out. */
GEMM_API gemm_status gemm_kernel_query(int32_t id, gemm_kernel_info *out);

/*
 * The choice gemm_f32 / gemm_bf16f32 would make for these arguments,
 * computed on the host without touching the GPU.  Pointers are only
 * inspected (NULL-ness and alignment), never dereferenced.  force_kernel = 0
 * lets the library choose; a positive id asks for that kernel and fails with
 * GEMM_ERR_UNSUPPORTED if it cannot run these operands (wrong dtype, or a
 * vector width the alignment does not allow, or a workspace kernel without
 * enough workspace).  workspace_bytes is the size a call would pass (0 for
 * none).  Returns the same status the call itself would return before
 * launching.
 */
GEMM_API gemm_status gemm_plan_query(int32_t dtype, int64_t M, int64_t N, int64_t K, float alpha,
                            const void *A, int64_t lda, const void *B, int64_t ldb,
                            float beta, const float *C, int64_t ldc,
                            int32_t force_kernel, int64_t workspace_bytes, gemm_plan *out);

/*
 * Fused epilogue ("Tiled matrix multiplication", section "Implementation
 * notes": bias, activation and scaling are applied while the tile is still
 * in registers, which saves a full read and write of C; "Efficiency",
 * epilogue fusion).  With an epilogue the call computes
 *
 *     C[i][j] = act(alpha * (A x B)[i][j] + beta * C0[i][j] + bias[j])
 *
 * bias: N floats (4-byte aligned device memory, read only), or NULL for no
 * bias.  activation: GEMM_ACT_NONE, GEMM_ACT_RELU (max(x, 0), NaN stays
 * NaN) or GEMM_ACT_GELU (x * Phi(x) with the normal CDF, erf form).  The
 * quick returns apply too: K == 0 or alpha == 0 gives act(beta*C0 + bias),
 * with C0 not read when beta == 0.  A NULL descriptor is the plain call.
 * Workspace arguments are those of gemm_f32_ws / gemm_bf16f32_ws (a K split
 * applies the epilogue once, in its reduce step).
 *
 * Output quantisation (the result converted in registers before it is
 * stored).  out_type GEMM_OUT_F32 (0) writes C as above.  GEMM_OUT_BF16 and
 * GEMM_OUT_FP8 write
 *
 *     out[i*ldo + j] = round(s * act(alpha * (A x B)[i][j] + beta * C0[i][j] + bias[j]))
 *
 * to `out` instead, with s = out_scale (0 is taken as 1), rounding to the
 * nearest value with ties to even: bfloat16 bit patterns (uint16_t; past the
 * largest finite value the rounding gives infinity) or OCP E4M3 bytes
 * (uint8_t; magnitudes from 448 up saturate to +-448, the format having no
 * infinities).  NaN stays NaN.  C is then not written; it is read as C0
 * only when beta != 0 and may be NULL otherwise.  out must be aligned to its
 * element size, ldo >= max(1, N).  A zero-filled descriptor (bias NULL,
 * activation and out_type 0) is the plain call.
 * Errors: GEMM_ERR_INVALID_ARG for an unknown activation or output type, a
 * misaligned bias or output, a NULL output or ldo < N, besides those of the
 * plain call.  GEMM_ERR_UNSUPPORTED when a forced kernel cannot write the
 * output type (gemm_kernel_info.outputs).
 */
typedef enum gemm_activation {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,
    GEMM_ACT_GELU = 2
} gemm_activation;

typedef enum gemm_output {
    GEMM_OUT_F32 = 0,        /* fp32, to C */
    GEMM_OUT_BF16 = 1,       /* bfloat16 bit patterns, to out */
    GEMM_OUT_FP8 = 2         /* OCP E4M3 bytes, saturating, to out */
} gemm_output;

typedef struct gemm_epilogue {
    const float *bias;       /* N floats or NULL */
    int32_t activation;      /* gemm_activation */
    int32_t out_type;        /* gemm_output */
    void *out;               /* GEMM_OUT_BF16 / GEMM_OUT_FP8: M x N output, row i at out + i*ldo */
    int64_t ldo;             /* elements between rows of out */
    float out_scale;         /* multiplies the result before rounding; 0 means 1 */
} gemm_epilogue;

GEMM_API gemm_status gemm_f32_epi(int64_t M, int64_t N, int64_t K, float alpha,
                                  const float *A, int64_t lda, const float *B, int64_t ldb,
                                  float beta, float *C, int64_t ldc, const gemm_epilogue *epilogue,
                                  void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

GEMM_API gemm_status gemm_bf16f32_epi(int64_t M, int64_t N, int64_t K, float alpha,
                                      const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                                      float beta, float *C, int64_t ldc, const gemm_epilogue *epilogue,
                                      void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

/*
 * gemm_f32_epi / gemm_bf16f32_epi with a forced kernel (force_kernel as in
 * gemm_plan_query; 0 lets the library choose), for tests and tuning.  A NULL
 * epilogue is the plain call, so with one these are gemm_f32_ws /
 * gemm_bf16f32_ws with a forced kernel.
 */
GEMM_API gemm_status gemm_f32_ex(int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb,
                        float beta, float *C, int64_t ldc,
                        int32_t force_kernel, const gemm_epilogue *epilogue,
                        void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

GEMM_API gemm_status gemm_bf16f32_ex(int64_t M, int64_t N, int64_t K, float alpha,
                            const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                            float beta, float *C, int64_t ldc,
                            int32_t force_kernel, const gemm_epilogue *epilogue,
                            void *workspace, int64_t workspace_bytes, gemm_stream_t stream);


/*
 * The general call: any operand type (gemm_dtype) and either layout of each
 * operand (gemm_op), with the optional fused epilogue, workspace and forced
 * kernel of gemm_f32_ex.  A and B point to fp32, bf16 (uint16_t) or fp8
 * E4M3 (uint8_t) elements as dtype says; C is fp32.  Every combination runs:
 *   - untransposed fp32 and bf16 take the kernels above;
 *   - M <= 16 with B transposed (GEMM_OP_T: B stored N x K, the layout of
 *     a linear layer's weights), any operand type, takes a streaming kernel
 *     that loads each weight row straight into the matrix instruction, when
 *     the rows of B are whole 16-byte chunks (aligned base, K and ldb) and,
 *     with A untransposed, so are A's; A stored K x M is gathered element
 *     by element (fp8 with a workspace takes the fp8 kernel below, split
 *     over K, where A's rows are whole 16-byte chunks);
 *   - fp32 and bf16 with M <= 16, A transposed and B untransposed (A
 *     stored K x M) take the streaming kernels of gemm_f32 and
 *     gemm_bf16f32, which then gather A's values from the rows of its
 *     stored transpose (bf16 with 16-byte loads when M and lda are
 *     multiples of 8 and A is 16-byte aligned, else 2-byte loads);
 *   - fp8 with M <= 16, both operands untransposed and no workspace takes a
 *     streaming kernel through byte-transposing LDS reads when N is at most
 *     128 * 128 (with a workspace the fp8 kernel below, split over K, is
 *     as fast); with A stored K x M it takes that kernel, loading A a byte
 *     a lane, whenever A's rows are not whole 16-byte chunks;
 *   - M == 1 with A transposed and lda == 1 (A stored K x 1, the same
 *     memory as a 1 x K row) runs as A untransposed unless a kernel is
 *     forced;
 *   - fp32 and bf16 with either operand transposed take the matrix-core
 *     kernel for that layout when the stored rows of A and B are whole
 *     16-byte chunks;
 *   - fp8 takes the fp8 matrix-core kernel for its layout when the stored
 *     rows of A and B (K, M or N long) and lda, ldb are whole 16-byte
 *     chunks on 16-byte aligned bases;
 *   - the rest take a general kernel that loads elements one by one and
 *     multiplies in fp32.
 *
 * fp8 accuracy.  Products of two E4M3 values are exact; the fp8 matrix core
 * sums each run of 8 consecutive k with truncation below 2^-13 of the run's
 * largest product, then adds the runs in fp32, so its error is at most
 * about 2^-10 * |alpha| * sum over runs of the largest |product| plus the
 * usual fp32 accumulation error.  Per-tensor scales fold into alpha.
 * Errors: GEMM_ERR_INVALID_ARG for an unknown dtype or op, besides those of
 * gemm_f32_ex.  A call with op_a == op_b == GEMM_OP_N and dtype fp32 or bf16
 * is exactly gemm_f32_ex / gemm_bf16f32_ex.
 */
GEMM_API gemm_status gemm_general(int32_t dtype, int32_t op_a, int32_t op_b,
                                  int64_t M, int64_t N, int64_t K, float alpha,
                                  const void *A, int64_t lda, const void *B, int64_t ldb,
                                  float beta, float *C, int64_t ldc,
                                  int32_t force_kernel, const gemm_epilogue *epilogue,
                                  void *workspace, int64_t workspace_bytes, gemm_stream_t stream);

/* gemm_plan_query with operand layouts: the plan gemm_general would take. */
GEMM_API gemm_status gemm_plan_query_general(int32_t dtype, int32_t op_a, int32_t op_b,
                                             int64_t M, int64_t N, int64_t K, float alpha,
                                             const void *A, int64_t lda, const void *B, int64_t ldb,
                                             float beta, const float *C, int64_t ldc,
                                             int32_t force_kernel, int64_t workspace_bytes,
                                             gemm_plan *out);

/*
 * gemm_general for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it).  The
 * arguments are those of gemm_general without the workspace: the K-split
 * paths keep their partial products in a static device array that the
 * library holds, GEMM_STATIC_SCRATCH_BYTES (32 MiB) on each GPU it is called
 * on, from the first call on that device until the process ends.  The call
 * allocates nothing itself; the result is the one gemm_general gives with a
 * workspace of that size.
 *
 * Limit: when gemm_workspace_size(dtype, M, N, K) exceeds
 * GEMM_STATIC_SCRATCH_BYTES the call returns GEMM_ERR_SCRATCH and does
 * nothing (pass a workspace to gemm_general instead).  Argument errors are
 * reported first, as by gemm_general.
 *
 * Sharing: all calls on one GPU use the same array.  It needs no clearing
 * (every partial product is written before it is read), but calls that can
 * overlap on one GPU (different streams not ordered by events, or several
 * host threads with no ordering) race on it.  Calls on one stream are
 * ordered and safe.
 */
#define GEMM_STATIC_SCRATCH_BYTES ((int64_t)32 << 20)

GEMM_API gemm_status gemm_general_noalloc(int32_t dtype, int32_t op_a, int32_t op_b,
                                          int64_t M, int64_t N, int64_t K, float alpha,
                                          const void *A, int64_t lda, const void *B, int64_t ldb,
                                          float beta, float *C, int64_t ldc,
                                          int32_t force_kernel, const gemm_epilogue *epilogue,
                                          gemm_stream_t stream);

/* gemm_plan_query_general with an epilogue (its output type narrows the
 * kernels that can run): the plan gemm_general would take with it. */
GEMM_API gemm_status gemm_plan_query_epi(int32_t dtype, int32_t op_a, int32_t op_b,
                                         int64_t M, int64_t N, int64_t K, float alpha,
                                         const void *A, int64_t lda, const void *B, int64_t ldb,
                                         float beta, const float *C, int64_t ldc,
                                         int32_t force_kernel, const gemm_epilogue *epilogue,
                                         int64_t workspace_bytes, gemm_plan *out);

/*
 * Per-shape tuning ("A GEMM Kernel, Step by Step", section "Six parameters,
 * found by search": the best tile configuration for a shape is not
 * derivable, so it is found by timing the candidates).
 *
 * gemm_autotune() times, on the caller's buffers and stream, every kernel
 * that can run this call (reps calls each after one untimed call, with and
 * without a K split when a workspace is given) and records the fastest in a
 * process-wide table keyed by dtype, layout (op_a, op_b), M, N, K, the
 * operands' widest vector width and whether a workspace is passed.  It
 * blocks until the timings are
 * done.  C is used as scratch: its contents afterwards are unspecified (with
 * beta != 0 every timed call updates it), so make the real call afterwards.
 * `out` receives the plan that calls of this kind now take.  reps: 1..1000.
 * Later calls with no forced kernel (and gemm_plan_query) use a recorded
 * choice whenever it can run the call; otherwise the built-in rules choose.
 * gemm_autotune() tunes untransposed operands; gemm_autotune_general()
 * takes any operand type and layout with the arguments of gemm_general()
 * (op_a, op_b as there), and its entries steer gemm_general() calls of the
 * same kind.
 * The table is guarded by a mutex; autotuning concurrently with calls on
 * other threads is safe, though the timings then include their load.
 *
 * gemm_tuning_save() writes the table as text, one line per entry, naming
 * kernels (not ids): "dtype op_a op_b M N K vec_a vec_b has_ws kernel split
 * ms" under a "# libgemm tuning table v2" header.  gemm_tuning_load() adds
 * the entries of such a file (entries naming unknown kernels, or kernels
 * for another operand type or layout, are skipped) and returns how many it
 * added, or -1 if the file cannot be read or parsed.  Files without the v2
 * header are read in the earlier format, without op_a op_b, as untransposed
 * entries.
 */
GEMM_API gemm_status gemm_autotune(int32_t dtype, int64_t M, int64_t N, int64_t K, float alpha,
                                   const void *A, int64_t lda, const void *B, int64_t ldb,
                                   float beta, float *C, int64_t ldc,
                                   void *workspace, int64_t workspace_bytes, int32_t reps,
                                   gemm_stream_t stream, gemm_plan *out);
GEMM_API gemm_status gemm_autotune_general(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N,
                                           int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                                           int64_t ldb, float beta, float *C, int64_t ldc, void *workspace,
                                           int64_t workspace_bytes, int32_t reps, gemm_stream_t stream,
                                           gemm_plan *out);
GEMM_API int32_t gemm_tuning_count(void);
GEMM_API void gemm_tuning_clear(void);
GEMM_API gemm_status gemm_tuning_save(const char *path);
GEMM_API int32_t gemm_tuning_load(const char *path);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_GEMM_H */
