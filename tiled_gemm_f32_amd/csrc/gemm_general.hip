// General GEMM for every operand type and layout: the kernel that runs what
// the faster kernels cannot (transposed operands, fp8 operands outside the
// layout of the fp8 ring kernel, operands with no 16-byte alignment).
//
// It is the blocked method of "Tiled matrix multiplication" ("How it
// works"): 128 x 128 output tiles, 16-deep k slices staged through LDS and
// double buffered, four waves each keeping a 64 x 64 accumulator tile in
// registers.  Every operand element is loaded on its own, lanes walking the
// operand's contiguous dimension for its layout (the coalescing rung of "A
// GEMM Kernel, Step by Step"); out-of-range elements are zero (page 1,
// section 3).  Values are widened exactly to fp32 (bf16 by a 16-bit shift,
// fp8 E4M3 by the hardware conversion) and stored in LDS in the orientation
// the matrix core reads, so one consume loop serves all layouts: products
// run on v_mfma_f32_32x32x2_f32, exact for all three operand types, and
// accumulate in fp32.
//
// Layouts (GemmParams::op_a / op_b): op_a == GEMM_OP_N reads A[m][k] at
// A + m*lda + k, GEMM_OP_T at A + k*lda + m; op_b == GEMM_OP_N reads
// B[k][n] at B + k*ldb + n, GEMM_OP_T at B + n*ldb + k.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

template <int DT> struct Elem;
template <> struct Elem<GEMM_DTYPE_F32> {
    typedef float T;
    static __device__ __forceinline__ float widen(const T *p, int64_t i) { return p[i]; }
};
template <> struct Elem<GEMM_DTYPE_BF16F32> {
    typedef uint16_t T;
    static __device__ __forceinline__ float widen(const T *p, int64_t i) {
        return __uint_as_float((uint32_t)p[i] << 16);
    }
};
template <> struct Elem<GEMM_DTYPE_FP8F32> {
    typedef uint8_t T;
    // OCP E4M3 on gfx950 (byte 0 of the source register).
    static __device__ __forceinline__ float widen(const T *p, int64_t i) {
        return __builtin_amdgcn_cvt_f32_fp8((int)p[i], 0);
    }
};

constexpr int kBM = 128, kBN = 128, kBK = 16, kThreads = 256;
constexpr int kAStride = kBK + 4;      // floats per LDS row of the A panel ([m][k])
constexpr int kBStride = kBN + 4;      // floats per LDS row of the B panel ([k][n])
constexpr int kPer = kBM * kBK / kThreads;   // elements of each panel per thread (8)
static_assert(kBM * kBK == kBK * kBN, "both panels split the same way");

// Panel coordinates of element i of this thread.  The fast index follows the
// operand's contiguous dimension in memory.
template <int OP>
__device__ __forceinline__ void a_coord(int tid, int i, int &r, int &kk) {
    const int c = tid + i * kThreads;
    if (OP == GEMM_OP_N) {
        r = c / kBK;
        kk = c % kBK;
    } else {
        kk = c / kBM;
        r = c % kBM;
    }
}
template <int OP>
__device__ __forceinline__ void b_coord(int tid, int i, int &kk, int &n) {
    const int c = tid + i * kThreads;
    if (OP == GEMM_OP_N) {
        kk = c / kBN;
        n = c % kBN;
    } else {
        n = c / kBK;
        kk = c % kBK;
    }
}

template <int DT, int OPA, int OPB>
__global__ void __launch_bounds__(kThreads)
general_kernel(GemmParams p, int tiles_m, int tiles_n) {
    typedef Elem<DT> E;
    typedef typename E::T T;
    apply_k_split<T>(p);

    __shared__ __attribute__((aligned(16))) float lds_a[2][kBM * kAStride];
    __shared__ __attribute__((aligned(16))) float lds_b[2][kBK * kBStride];

    const int tid = threadIdx.x;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    const T *A = static_cast<const T *>(p.A);
    const T *B = static_cast<const T *>(p.B);

    float sa[kPer], sb[kPer];
    auto fetch = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int r, kk;
            a_coord<OPA>(tid, i, r, kk);
            const int gm = m0 + r, gk = k0 + kk;
            const int64_t idx = OPA == GEMM_OP_N ? gm * lda + gk : gk * lda + gm;
            sa[i] = (gm < M && gk < K) ? E::widen(A, idx) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int kk, n;
            b_coord<OPB>(tid, i, kk, n);
            const int gk = k0 + kk, gn = n0 + n;
            const int64_t idx = OPB == GEMM_OP_N ? gk * ldb + gn : gn * ldb + gk;
            sb[i] = (gk < K && gn < N) ? E::widen(B, idx) : 0.0f;
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int r, kk;
            a_coord<OPA>(tid, i, r, kk);
            lds_a[buf][r * kAStride + kk] = sa[i];
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int kk, n;
            b_coord<OPB>(tid, i, kk, n);
            lds_b[buf][kk * kBStride + n] = sb[i];
        }
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // Lane (row l32, half h) holds k = 8h .. 8h + 7 of its A rows and of its B
    // columns; each matrix instruction takes one k from each lane half.
    auto consume = [&](int buf) {
        float af[2][8];
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
            const float *src = &lds_a[buf][(wm * 64 + 32 * fm + l32) * kAStride + 8 * h];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 4 * q);
                af[fm][4 * q + 0] = v.x;
                af[fm][4 * q + 1] = v.y;
                af[fm][4 * q + 2] = v.z;
                af[fm][4 * q + 3] = v.w;
            }
        }
        const float *bsrc = &lds_b[buf][8 * h * kBStride + wn * 64 + l32];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float b0 = bsrc[s * kBStride], b1 = bsrc[s * kBStride + 32];
#pragma unroll
            for (int fm = 0; fm < 2; ++fm) {
                acc[fm][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[fm][s], b0, acc[fm][0], 0, 0, 0);
                acc[fm][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[fm][s], b1, acc[fm][1], 0, 0, 0);
            }
        }
    };

    const int nk = (K + kBK - 1) / kBK;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) fetch(kt + 1);
        consume(cur);
        if (more) stash(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Fragment register r of lane (h, l32) is row 8*(r/4) + 4*h + r%4,
    // column l32 of its 32 x 32 block.
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
            const int col = n0 + wn * 64 + 32 * fn + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + 32 * fm + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) {
                    float v = alpha * acc[fm][fn][r];
                    if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)row * p.ldc + col], v);
                    store_out_any(p, row, col, epilogue_value(v, col, p.bias, p.act));
                }
            }
        }
    }
}

template <int DT>
hipError_t launch_general(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + kBM - 1) / kBM, tiles_n = (p.N + kBN - 1) / kBN;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const void *fn;
    if (p.op_a == GEMM_OP_N)
        fn = p.op_b == GEMM_OP_N ? reinterpret_cast<const void *>(&general_kernel<DT, GEMM_OP_N, GEMM_OP_N>)
                                 : reinterpret_cast<const void *>(&general_kernel<DT, GEMM_OP_N, GEMM_OP_T>);
    else
        fn = p.op_b == GEMM_OP_N ? reinterpret_cast<const void *>(&general_kernel<DT, GEMM_OP_T, GEMM_OP_N>)
                                 : reinterpret_cast<const void *>(&general_kernel<DT, GEMM_OP_T, GEMM_OP_T>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(kThreads), argv, 0,
                           stream);
}

// Explicit instantiations for the device pass (the table below is host-only).
#define GENERAL_INSTANCES(DT)                                                        \
    template __global__ void general_kernel<DT, GEMM_OP_N, GEMM_OP_N>(GemmParams, int, int); \
    template __global__ void general_kernel<DT, GEMM_OP_N, GEMM_OP_T>(GemmParams, int, int); \
    template __global__ void general_kernel<DT, GEMM_OP_T, GEMM_OP_N>(GemmParams, int, int); \
    template __global__ void general_kernel<DT, GEMM_OP_T, GEMM_OP_T>(GemmParams, int, int);
GENERAL_INSTANCES(GEMM_DTYPE_F32)
GENERAL_INSTANCES(GEMM_DTYPE_BF16F32)
GENERAL_INSTANCES(GEMM_DTYPE_FP8F32)

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// Last in the dispatcher's order: a call takes these only when no faster
// kernel runs its operands.
const KernelDesc kGeneralKernels[] = {
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, kBM, kBN, kBK, kThreads, 1, 1, "f32_general_128x128x16",
     &launch_general<GEMM_DTYPE_F32>, 0, nullptr, kLayoutAll, true, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, kBM, kBN, kBK, kThreads, 1, 1, "bf16_general_128x128x16",
     &launch_general<GEMM_DTYPE_BF16F32>, 0, nullptr, kLayoutAll, true, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, kBM, kBN, kBK, kThreads, 1, 1, "fp8_general_128x128x16",
     &launch_general<GEMM_DTYPE_FP8F32>, 0, nullptr, kLayoutAll, true, kOutAll},
};
const int kGeneralKernelCount = sizeof(kGeneralKernels) / sizeof(kGeneralKernels[0]);
#endif

}  // namespace gemm
