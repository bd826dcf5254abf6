// Internal interface between the C ABI (gemm_api.cpp) and the kernel files.
// Not installed; callers use include/gemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace gemm {

// Arguments of one GEMM launch, already validated by the host code:
// 0 < M, N, K < 2^31, lda and ldb below 2^31 elements, every panel or slice
// the chosen kernel reads through one buffer resource below 2^31 bytes
// (gemm_api.cpp, operands_fit), pointers aligned to their element size.  A and B are fp32, bf16 or fp8 according
// to the kernel; C is always fp32.  op_a / op_b are gemm_op layouts; a
// kernel runs only the layouts its table row lists.
struct GemmParams {
    const void *A;
    const void *B;
    float *C;
    int32_t M, N, K;
    int32_t lda, ldb;
    int64_t ldc;
    float alpha, beta;
    int32_t op_a, op_b;
    // K split (0: none).  With kchunk > 0 the tiled kernels run on a grid of
    // (tiles, ceil(K / kchunk)) workgroups; row y of the grid multiplies the
    // k range [y*kchunk, min(K, (y+1)*kchunk)) and stores that partial product
    // (alpha 1, beta 0) to partials + y*M*N with leading dimension N.
    int32_t kchunk;
    float *partials;
    // Fused epilogue: C = act(alpha * acc + beta * C0 + bias[column]); bias
    // may be null, act is a gemm_activation.
    const float *bias;
    int32_t act;
    // Output (gemm_output).  GEMM_OUT_F32 stores to C (out == C, ldo ==
    // ldc); the others store round(out_scale * value) to out, bf16 or E4M3,
    // and leave C unwritten (it is read as C0 when beta != 0).  Kernels run
    // only the outputs their table row lists.
    int32_t out_type;
    float out_scale;
    void *out;
    int64_t ldo;
};

inline int k_splits(const GemmParams &p) { return p.kchunk > 0 ? (p.K + p.kchunk - 1) / p.kchunk : 1; }
// Output type a launch stores: a K-split slice stores fp32 partials whatever
// the call's output (the reduce converts); kernels templated on the output
// type launch the matching instantiation.
inline int launch_out_type(const GemmParams &p) { return p.kchunk > 0 ? GEMM_OUT_F32 : p.out_type; }
// Most K slices the reduce kernel adds (every split path stays within it).
constexpr int kMaxReduceSplits = 16;

typedef hipError_t (*LaunchFn)(const GemmParams &p, hipStream_t stream);

// Operand layouts a kernel runs: bit 2*op_a + op_b.
constexpr int32_t kLayoutNN = 1, kLayoutNT = 2, kLayoutTN = 4, kLayoutTT = 8, kLayoutAll = 15;
// Output-type bits (bit gemm_output).
constexpr int32_t kOutF32 = 1, kOutAll = 7;

// C = alpha * (sum of the k_splits(p) partial products, in split order) +
// beta * C, for the tiled kernels' K split (defined with the skinny kernels).
hipError_t launch_splitk_reduce(const GemmParams &p, hipStream_t stream);
typedef hipError_t (*LaunchWsFn)(const GemmParams &p, void *workspace, hipStream_t stream);

// One row of the kernel table.
struct KernelDesc {
    int32_t dtype;     // gemm_dtype
    int32_t path;      // gemm_path
    int32_t tile_m, tile_n, tile_k;
    int32_t threads;
    int32_t vec_a, vec_b;
    const char *name;
    LaunchFn launch;
    int32_t min_k;     // the automatic choice skips this kernel below this K (0: no limit)
    LaunchWsFn launch_ws;  // set instead of `launch` for kernels that need the caller's workspace
    int32_t layouts = kLayoutNN;
    bool fallback = false;     // chosen only when no other kernel runs the call
    int32_t outputs = kOutF32;
};

// Split-K skinny kernel sizing, shared by its launcher and the workspace query:
// double the number of K slices (at most 8, each at least 512 deep) until
// strips * slices covers the 256 compute units.
inline int skinny_splits(int strips, int K) {
    int s = 1;
    while (s < 8 && strips * s < 256 && K / (2 * s) >= 512) s *= 2;
    return s;
}
// Workspace of the split-K skinny path: `splits` partial M x N fp32
// results, split-major.  One split needs none (the kernel finishes C itself).
inline int64_t skinny_workspace_bytes(int strips, int M, int N, int K) {
    const int s = skinny_splits(strips, K);
    return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

// Tables exported by the kernel files (constant-initialised).
extern const KernelDesc kF32TiledKernels[];
extern const int kF32TiledKernelCount;
extern const KernelDesc kBf16TiledKernels[];
extern const int kBf16TiledKernelCount;
extern const KernelDesc kF32SkinnyKernels[];
extern const int kF32SkinnyKernelCount;
extern const KernelDesc kF32SplitKernels[];
extern const int kF32SplitKernelCount;
extern const KernelDesc kFp8TiledKernels[];
extern const int kFp8TiledKernelCount;
extern const KernelDesc kGeneralKernels[];
extern const int kGeneralKernelCount;
extern const KernelDesc kBf16SplitKernels[];
extern const int kBf16SplitKernelCount;
extern const KernelDesc kSkinnyNtKernels[];
extern const int kSkinnyNtKernelCount;
extern const KernelDesc kBf16LinesKernels[];
extern const int kBf16LinesKernelCount;
extern const KernelDesc kFp8LinesKernels[];
extern const int kFp8LinesKernelCount;
extern const KernelDesc kFp8SkinnyKernels[];
extern const int kFp8SkinnyKernelCount;

// Size of the library's static device scratch (gemm_scratch.hip), the
// workspace of gemm_general_noalloc.
constexpr int64_t kStaticScratchBytes = int64_t(32) << 20;
// Device address of the current device's copy of that scratch (looked up
// once per device).
hipError_t static_scratch(void **ptr);

// The K == 0 / alpha == 0 result over p's M x N view: act(beta * C + bias)
// (C not read when beta == 0), stored as p's output type.
hipError_t launch_scale_c(const GemmParams &p, hipStream_t stream);

}  // namespace gemm
