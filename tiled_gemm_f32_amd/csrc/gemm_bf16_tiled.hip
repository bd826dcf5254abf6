// bf16-operand, fp32-accumulate blocked GEMM on the gfx950 matrix cores.
//
// Same blocking as the fp32 kernel (workgroup tile, double-buffered LDS
// panels, wave tiles of matrix-core fragments, fused alpha/beta epilogue;
// "Tiled matrix multiplication", section "How it works", down to its
// tensor-core level), with v_mfma_f32_32x32x16_bf16 fragments: each lane
// feeds 8 consecutive k values of one row of A and of one column of B.
//
// LDS layout.  Both panels are stored k-contiguous in 16-byte chunks of 8
// bf16: A as [BM][BK] (its natural row-major order) and B transposed as
// [BN][BK], so every fragment read is one 16-byte LDS load.  B arrives from
// HBM row-major (n contiguous); each thread fetches an 8 x 8 block (8 rows of
// 16 bytes, coalesced along n across lanes) and transposes it in registers
// before writing 8 chunks.  This is the page's "store one operand transposed"
// trick ("Tiled matrix multiplication", "Implementation notes"; "A GEMM
// Kernel, Step by Step", rung six) applied to B, the operand the matrix core
// wants transposed here.  Chunk columns are XOR-swizzled by row so that the
// 16 lanes served together by the LDS land on distinct banks, instead of
// padding (the bank-conflict item of "What is left").
//
// bf16 x bf16 products are exact in fp32; all sums are fp32.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

template <int BM, int BN, int BK, int WM, int WN>
struct Bf16Tiled {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int kFragM = kWaveM / 32;
    static constexpr int kFragN = kWaveN / 32;
    static constexpr int kSteps = BK / 16;            // MFMA k-steps per slice
    static constexpr int kChunks = BK / 8;            // 16-byte chunks per LDS row
    static constexpr int kAChunkCount = BM * kChunks;
    static constexpr int kAPer = kAChunkCount / kThreads;
    // B is transposed in blocks of kKR k-rows x 8 n-columns, one block per
    // thread per slice: 8 rows when there are enough blocks to go round,
    // else 4 (each column then fills half a 16-byte chunk).
    static constexpr int kKR = ((BK / 8) * (BN / 8) >= kThreads) ? 8 : 4;
    static constexpr int kBBlocks = (BK / kKR) * (BN / 8);
    static constexpr int kBPer = kBBlocks / kThreads;

    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be whole 32x32 fragments");
    static_assert(kChunks == 8, "swizzle below assumes 8 chunks (128 bytes) per LDS row");
    static_assert(kAChunkCount % kThreads == 0, "A panel must split evenly");
    static_assert(kBPer >= 1 && kBBlocks % kThreads == 0, "B panel must split evenly");
};

// Physical chunk of logical chunk `ch` in LDS row `row`.
__device__ __forceinline__ int swz(int row, int ch) { return ch ^ ((row >> 1) & 7); }

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
__global__ void __launch_bounds__(64 * WM * WN)
bf16_tiled_kernel(GemmParams p, int tiles_m, int tiles_n) {
    typedef Bf16Tiled<BM, BN, BK, WM, WN> Cfg;

    __shared__ __attribute__((aligned(16))) u32x4 lds_a[2][BM * Cfg::kChunks];
    __shared__ __attribute__((aligned(16))) u32x4 lds_b[2][BN * Cfg::kChunks];

    const int tid = threadIdx.x;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;

    const uint16_t *a_panel = static_cast<const uint16_t *>(p.A) + (int64_t)m0 * lda;
    const int a_rows = min(BM, M - m0);
    const rsrc_t ra = make_rsrc(a_panel, clamp_extent(((int64_t)(a_rows - 1) * lda + K) * 2));

    // A chunk c: row c / kChunks, logical chunk c % kChunks (8 lanes per 128-byte row).
    uint32_t a_off[Cfg::kAPer];
    int a_k[Cfg::kAPer], a_lds[Cfg::kAPer];
#pragma unroll
    for (int i = 0; i < Cfg::kAPer; ++i) {
        const int c = tid + i * Cfg::kThreads;
        const int r = c / Cfg::kChunks, ch = c % Cfg::kChunks;
        a_off[i] = (uint32_t)(r * lda + ch * 8) * 2u;
        a_k[i] = ch * 8;
        a_lds[i] = r * Cfg::kChunks + swz(r, ch);
    }
    // B block b: k rows KR*kg .. KR*kg+KR-1, n columns 8*ng .. 8*ng+7 of the slice.
    constexpr int KR = Cfg::kKR;
    uint32_t b_off[Cfg::kBPer];
    int b_kg[Cfg::kBPer], b_ng[Cfg::kBPer];
#pragma unroll
    for (int i = 0; i < Cfg::kBPer; ++i) {
        const int b = tid + i * Cfg::kThreads;
        const int kg = b / (BN / 8), ng = b % (BN / 8);
        b_off[i] = (uint32_t)(KR * kg * ldb + 8 * ng) * 2u;
        b_kg[i] = kg;
        b_ng[i] = ng;
    }

    u32x4 sa[Cfg::kAPer];
    u32x4 sb[Cfg::kBPer][KR];

    auto fetch = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < Cfg::kAPer; ++i) {
            if constexpr (VA == 8) {
                const uint32_t off = (k0 + a_k[i] < K) ? a_off[i] + (uint32_t)k0 * 2u : kOutOfRange;
                sa[i] = load_b128(ra, off);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t o0 = (k0 + a_k[i] + e < K) ? a_off[i] + (uint32_t)(k0 + e) * 2u : kOutOfRange;
                    const uint32_t o1 = (k0 + a_k[i] + e + 1 < K) ? a_off[i] + (uint32_t)(k0 + e + 1) * 2u : kOutOfRange;
                    w[e / 2] = (uint32_t)load_b16(ra, o0) | ((uint32_t)load_b16(ra, o1) << 16);
                }
                sa[i] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        // Rows at or past K fall outside the slice's extent and read as zero;
        // columns past N only feed outputs that are never stored.
        const uint16_t *b_slice = static_cast<const uint16_t *>(p.B) + (int64_t)k0 * ldb + n0;
        const rsrc_t rb = make_rsrc(b_slice, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
#pragma unroll
        for (int i = 0; i < Cfg::kBPer; ++i) {
#pragma unroll
            for (int e = 0; e < KR; ++e) {
                const uint32_t off = b_off[i] + (uint32_t)(e * ldb) * 2u;
                if constexpr (VB == 8) {
                    sb[i][e] = load_b128(rb, off);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[q] = (uint32_t)load_b16(rb, off + 4u * q) | ((uint32_t)load_b16(rb, off + 4u * q + 2u) << 16);
                    sb[i][e] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        }
    };

    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Cfg::kAPer; ++i) lds_a[buf][a_lds[i]] = sa[i];
#pragma unroll
        for (int i = 0; i < Cfg::kBPer; ++i) {
            // sb[i][e] word w holds columns (2w, 2w+1) of k row e.  Column c of
            // the transposed block needs, in word q, rows (2q, 2q+1) of column c.
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint32_t w[KR / 2];
#pragma unroll
                for (int q = 0; q < KR / 2; ++q) {
                    const uint32_t lo = sb[i][2 * q][c >> 1], hi = sb[i][2 * q + 1][c >> 1];
                    w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                const int row = 8 * b_ng[i] + c;
                if constexpr (KR == 8) {
                    lds_b[buf][row * Cfg::kChunks + swz(row, b_kg[i])] = u32x4{w[0], w[1], w[2], w[3]};
                } else {
                    // Half chunk: k group kg covers half (kg & 1) of logical chunk kg / 2.
                    u32x2 *dst = reinterpret_cast<u32x2 *>(&lds_b[buf][row * Cfg::kChunks + swz(row, b_kg[i] >> 1)]);
                    dst[b_kg[i] & 1] = u32x2{w[0], w[1]};
                }
            }
        }
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
#pragma unroll
        for (int s = 0; s < Cfg::kSteps; ++s) {
            // Lane (row l32, half h) supplies k = 16*s + 8*h .. 16*s + 8*h + 7.
            const int ch = 2 * s + h;
            bf16x8 af[Cfg::kFragM], bfr[Cfg::kFragN];
#pragma unroll
            for (int fm = 0; fm < Cfg::kFragM; ++fm) {
                const int row = wm * Cfg::kWaveM + 32 * fm + l32;
                af[fm] = __builtin_bit_cast(bf16x8, lds_a[buf][row * Cfg::kChunks + swz(row, ch)]);
            }
#pragma unroll
            for (int fn = 0; fn < Cfg::kFragN; ++fn) {
                const int row = wn * Cfg::kWaveN + 32 * fn + l32;
                bfr[fn] = __builtin_bit_cast(bf16x8, lds_b[buf][row * Cfg::kChunks + swz(row, ch)]);
            }
#pragma unroll
            for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
                for (int fn = 0; fn < Cfg::kFragN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
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
hipError_t launch_bf16_tiled(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&bf16_tiled_kernel<BM, BN, BK, WM, WN, VA, VB, GROUP_M>),
                           dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * WM * WN), argv, 0, stream);
}

#define BF16_TILED(BM, BN, BK, WM, WN, VA, VB, G)                                             \
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, BM, BN, BK, 64 * WM * WN, VA, VB,                   \
     "bf16_mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_a" #VA "b" #VB,                    \
     &launch_bf16_tiled<BM, BN, BK, WM, WN, VA, VB, G>}

// Explicit instantiations: the device pass never sees the host-only table
// below, so the kernels it needs are named here.
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 8, 8, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 8, 1, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 1, 8, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 1, 1, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 8, 8, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 8, 1, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 1, 8, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 1, 1, 8>(GemmParams, int, int);

}  // namespace

// The table holds host function pointers, so it exists only in the host pass.
#if !defined(__HIP_DEVICE_COMPILE__)
const KernelDesc kBf16TiledKernels[] = {
    BF16_TILED(256, 256, 64, 2, 2, 8, 8, 4),
    BF16_TILED(256, 256, 64, 2, 2, 8, 1, 4),
    BF16_TILED(256, 256, 64, 2, 2, 1, 8, 4),
    BF16_TILED(256, 256, 64, 2, 2, 1, 1, 4),
    BF16_TILED(128, 128, 64, 2, 2, 8, 8, 8),
    BF16_TILED(128, 128, 64, 2, 2, 8, 1, 8),
    BF16_TILED(128, 128, 64, 2, 2, 1, 8, 8),
    BF16_TILED(128, 128, 64, 2, 2, 1, 1, 8),
};
const int kBf16TiledKernelCount = sizeof(kBf16TiledKernels) / sizeof(kBf16TiledKernels[0]);
#endif

}  // namespace gemm
