// fp32 blocked GEMM on the gfx950 matrix cores.
//
// The structure is the blocked method the pages build up ("Tiled matrix
// multiplication", section "How it works"; "A GEMM Kernel, Step by Step",
// rungs three to six and "The last rung"), mapped onto CDNA4:
//
//   * C is cut into BM x BN workgroup tiles (one workgroup per tile), walked
//     in an XCD-aware grouped order (gemm_device.hpp).
//   * For each BK-deep slice of k the workgroup cooperatively copies a
//     BM x BK panel of A and a BK x BN panel of B from HBM into LDS.  Lanes
//     walk the contiguous dimension of each operand (the coalescing rung)
//     with 16-byte loads when alignment allows (the float4 rung), and
//     out-of-range elements arrive as zero (the edge handling of page 1,
//     section 3).
//   * LDS is double-buffered: the next slice is fetched into registers while
//     the current one is consumed, then written to the other buffer, so one
//     barrier per slice suffices (the double-buffering item of "What is
//     left").  Panel rows are padded by 4 floats to spread lanes over banks.
//   * The block tile is split among 4 wavefronts (the warp tile of "The last
//     rung"); each wave keeps its whole output sub-tile in accumulator
//     registers as 32 x 32 fragments of v_mfma_f32_32x32x2_f32, which
//     replaces the per-thread TM x TN register micro-tile: one instruction
//     performs 2048 multiply-adds from one A and one B value per lane.
//   * The epilogue applies C = alpha * acc + beta * C0 in registers and
//     stores only in-range entries (masked store).
//
// Reduction order within each output: k slices in order; inside a slice the
// matrix core sums pairs of k values, lane half h taking k in
// [h*BK/2, (h+1)*BK/2).  Any order is a correct evaluation of the sum; the
// result is deterministic run to run.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

template <int V> struct F32Chunk;
template <> struct F32Chunk<4> {
    typedef u32x4 T;
    static __device__ __forceinline__ T load(rsrc_t r, uint32_t off) { return load_b128(r, off); }
    static __device__ __forceinline__ void store(float *dst, T v) { *reinterpret_cast<u32x4 *>(dst) = v; }
};
template <> struct F32Chunk<1> {
    typedef uint32_t T;
    static __device__ __forceinline__ T load(rsrc_t r, uint32_t off) { return load_b32(r, off); }
    static __device__ __forceinline__ void store(float *dst, T v) { *reinterpret_cast<uint32_t *>(dst) = v; }
};

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
struct F32Tiled {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int kFragM = kWaveM / 32;
    static constexpr int kFragN = kWaveN / 32;
    static constexpr int kHalfK = BK / 2;
    static constexpr int kAStride = BK + 4;   // floats per LDS row of the A panel
    static constexpr int kBStride = BN + 4;   // floats per LDS row of the B panel
    static constexpr int kAPer = BM * BK / VA / kThreads;
    static constexpr int kBPer = BK * BN / VB / kThreads;
    static constexpr int kALds = BM * kAStride;
    static constexpr int kBLds = BK * kBStride;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 fragments");
    static_assert(BM * BK % (VA * kThreads) == 0, "A panel must split evenly over threads");
    static_assert(BK * BN % (VB * kThreads) == 0, "B panel must split evenly over threads");
    static_assert(kHalfK % 4 == 0, "each lane half reads whole 16-byte groups of k");
};

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
__global__ void __launch_bounds__(64 * WM * WN)
f32_tiled_kernel(GemmParams p, int tiles_m, int tiles_n) {
    typedef F32Tiled<BM, BN, BK, WM, WN, VA, VB, GROUP_M> Cfg;
    typedef F32Chunk<VA> CA;
    typedef F32Chunk<VB> CB;

    __shared__ __attribute__((aligned(16))) float lds_a[2][Cfg::kALds];
    __shared__ __attribute__((aligned(16))) float lds_b[2][Cfg::kBLds];

    const int tid = threadIdx.x;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;

    // A row panel: its extent ends right after the last valid element, so rows
    // at or past M read as zero.  lda < 2^21 keeps every offset below 2^31.
    const float *a_panel = static_cast<const float *>(p.A) + (int64_t)m0 * lda;
    const int a_rows = min(BM, M - m0);
    const rsrc_t ra = make_rsrc(a_panel, clamp_extent(((int64_t)(a_rows - 1) * lda + K) * 4));

    uint32_t a_off[Cfg::kAPer];
    int a_k[Cfg::kAPer], a_lds[Cfg::kAPer];
#pragma unroll
    for (int i = 0; i < Cfg::kAPer; ++i) {
        const int c = tid + i * Cfg::kThreads;
        const int r = c / (BK / VA), kc = (c % (BK / VA)) * VA;
        a_off[i] = (uint32_t)(r * lda + kc) * 4u;
        a_k[i] = kc;
        a_lds[i] = r * Cfg::kAStride + kc;
    }
    uint32_t b_off[Cfg::kBPer];
    int b_lds[Cfg::kBPer];
#pragma unroll
    for (int i = 0; i < Cfg::kBPer; ++i) {
        const int c = tid + i * Cfg::kThreads;
        const int r = c / (BN / VB), nc = (c % (BN / VB)) * VB;
        b_off[i] = (uint32_t)(r * ldb + nc) * 4u;
        b_lds[i] = r * Cfg::kBStride + nc;
    }

    typename CA::T sa[Cfg::kAPer];
    typename CB::T sb[Cfg::kBPer];

    auto fetch = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < Cfg::kAPer; ++i) {
            // Columns at or past K hold the next row (or padding): force zero.
            const uint32_t off = (k0 + a_k[i] < K) ? a_off[i] + (uint32_t)k0 * 4u : kOutOfRange;
            sa[i] = CA::load(ra, off);
        }
        // B slice: rebased per slice so offsets stay small; rows at or past K
        // fall outside the extent and read as zero.
        const float *b_slice = static_cast<const float *>(p.B) + (int64_t)k0 * ldb + n0;
        const rsrc_t rb = make_rsrc(b_slice, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 4));
#pragma unroll
        for (int i = 0; i < Cfg::kBPer; ++i) sb[i] = CB::load(rb, b_off[i]);
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Cfg::kAPer; ++i) CA::store(&lds_a[buf][a_lds[i]], sa[i]);
#pragma unroll
        for (int i = 0; i < Cfg::kBPer; ++i) CB::store(&lds_b[buf][b_lds[i]], sb[i]);
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, l32 = lane & 31;

    f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j) acc[i][j] = f32x16{};

    auto consume = [&](int buf) {
        // A fragments: lane (row l32, half h) holds k = h*BK/2 .. h*BK/2 + BK/2 - 1.
        float af[Cfg::kFragM][Cfg::kHalfK];
#pragma unroll
        for (int fm = 0; fm < Cfg::kFragM; ++fm) {
            const float *src = &lds_a[buf][(wm * Cfg::kWaveM + 32 * fm + l32) * Cfg::kAStride + h * Cfg::kHalfK];
#pragma unroll
            for (int q = 0; q < Cfg::kHalfK / 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 4 * q);
                af[fm][4 * q + 0] = v.x;
                af[fm][4 * q + 1] = v.y;
                af[fm][4 * q + 2] = v.z;
                af[fm][4 * q + 3] = v.w;
            }
        }
        const float *bsrc = &lds_b[buf][h * Cfg::kHalfK * Cfg::kBStride + wn * Cfg::kWaveN + l32];
#pragma unroll
        for (int s = 0; s < Cfg::kHalfK; ++s) {
            float bv[Cfg::kFragN];
#pragma unroll
            for (int fn = 0; fn < Cfg::kFragN; ++fn) bv[fn] = bsrc[s * Cfg::kBStride + 32 * fn];
#pragma unroll
            for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
                for (int fn = 0; fn < Cfg::kFragN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[fm][s], bv[fn], acc[fm][fn], 0, 0, 0);
        }
    };

    const int nk = (K + BK - 1) / BK;
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
    for (int fm = 0; fm < Cfg::kFragM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < Cfg::kFragN; ++fn) {
            const int col = n0 + wn * Cfg::kWaveN + 32 * fn + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * Cfg::kWaveM + 32 * fm + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) {
                    float *cp = p.C + (int64_t)row * p.ldc + col;
                    float v = alpha * acc[fm][fn][r];
                    if (beta != 0.0f) v = fmaf(beta, *cp, v);
                    *cp = v;
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
hipError_t launch_f32_tiled(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&f32_tiled_kernel<BM, BN, BK, WM, WN, VA, VB, GROUP_M>),
                           dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WM * WN), argv, 0, stream);
}

#define F32_TILED(BM, BN, BK, WM, WN, VA, VB, G)                                              \
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, BM, BN, BK, 64 * WM * WN, VA, VB,                       \
     "f32_mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_a" #VA "b" #VB,                     \
     &launch_f32_tiled<BM, BN, BK, WM, WN, VA, VB, G>}

// Explicit instantiations: the device pass never sees the host-only table
// below, so the kernels it needs are named here.
template __global__ void f32_tiled_kernel<256, 256, 16, 2, 2, 4, 4, 4>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<256, 256, 16, 2, 2, 4, 1, 4>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<256, 256, 16, 2, 2, 1, 4, 4>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<256, 256, 16, 2, 2, 1, 1, 4>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<128, 128, 16, 2, 2, 4, 4, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<128, 128, 16, 2, 2, 4, 1, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<128, 128, 16, 2, 2, 1, 4, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<128, 128, 16, 2, 2, 1, 1, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<64, 64, 16, 2, 2, 4, 4, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<64, 64, 16, 2, 2, 4, 1, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<64, 64, 16, 2, 2, 1, 4, 8>(GemmParams, int, int);
template __global__ void f32_tiled_kernel<64, 64, 16, 2, 2, 1, 1, 8>(GemmParams, int, int);

}  // namespace

// The table holds host function pointers, so it exists only in the host pass.
#if !defined(__HIP_DEVICE_COMPILE__)
// Order matters: the dispatcher takes the first kernel of the chosen tile
// shape whose vector widths the operands allow, so wider loads come first.
const KernelDesc kF32TiledKernels[] = {
    F32_TILED(256, 256, 16, 2, 2, 4, 4, 4),
    F32_TILED(256, 256, 16, 2, 2, 4, 1, 4),
    F32_TILED(256, 256, 16, 2, 2, 1, 4, 4),
    F32_TILED(256, 256, 16, 2, 2, 1, 1, 4),
    F32_TILED(128, 128, 16, 2, 2, 4, 4, 8),
    F32_TILED(128, 128, 16, 2, 2, 4, 1, 8),
    F32_TILED(128, 128, 16, 2, 2, 1, 4, 8),
    F32_TILED(128, 128, 16, 2, 2, 1, 1, 8),
    F32_TILED(64, 64, 16, 2, 2, 4, 4, 8),
    F32_TILED(64, 64, 16, 2, 2, 4, 1, 8),
    F32_TILED(64, 64, 16, 2, 2, 1, 4, 8),
    F32_TILED(64, 64, 16, 2, 2, 1, 1, 8),
};
const int kF32TiledKernelCount = sizeof(kF32TiledKernels) / sizeof(kF32TiledKernels[0]);
#endif

}  // namespace gemm
