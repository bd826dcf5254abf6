// fp8 (OCP E4M3) GEMM on the gfx950 matrix cores, fp32 accumulate and
// output; first for A untransposed (M x K) times B transposed (stored N x K),
// then for every other layout.
//
// With both operands stored k-contiguous, this is the bf16 ring kernel with
// both panels handled the way it handles A ("Tiled matrix multiplication",
// "How it works", at the tensor-core level; "A GEMM Kernel, Step by Step",
// "What is left": asynchronous copies into a multi-stage ring).  The fp8
// product instruction v_mfma_f32_32x32x64_f8f6f4 takes 64 k per call, so a
// 64-byte k slice of a row feeds exactly one instruction per fragment pair:
// the same bytes and the same 64 matrix cycles per slice as the bf16 kernel,
// for twice the multiply-adds.
//
//   Both slices: [256 rows][4 chunks of 16 B] (k contiguous),
//     chunk ^= (row >> 2) & 3 (the A layout of the bf16 ring, measured free
//     of bank conflicts there; the reads below have the same pattern).
//   Fragments: lane (h, l32) of a 32-row fragment holds bytes 32h .. 32h+31
//     of its row's slice (k = 32h .. 32h+31), read as two 16-byte ds_read_b128.
//     The instruction pairs byte b of an A lane with byte b of the B lane of
//     the same half, whatever its internal k order, so equal placement on
//     both sides gives the dot product.  It sums each run of 8 bytes (8
//     consecutive k here) at reduced precision before adding runs in fp32.
//
// Operands stored the other way (A as K x M, B as K x N: AKN, BKN) are
// contiguous along m or n instead of k.  Their slices are [64 k rows][256
// columns] of bytes, 16-byte chunk c of row k stored at chunk c ^ 2*(k % 8),
// loaded one whole 256-byte row per 16 lanes.  A fragment is gathered with
// ds_read_b64_tr_b8, which returns to lane j of a 16-lane group byte j % 8
// of the 8-byte reads of lanes (j / 8) + {0, 2, 4, 6, 8, 10, 12, 14}
// (probed): pointing those lanes at rows kb + 0 .. kb + 7 and the two halves
// of a 16-byte chunk gives each lane 8 consecutive k of one column, and four
// reads give the 32 consecutive k of the k-contiguous fragment, in the same
// byte order.  The swizzle puts each half-wave's 16 rows-and-chunks in 16
// different chunk columns, so the reads are free of bank conflicts.
//
// Schedule, per slice kt (stage kt % NS, register set kt % 2): every wave
// waits for its own reads of slice kt and for slice kt+1 to land, then a
// barrier; then 16 matrix instructions on slice kt, each paired with one of
// the 16 fragment reads of slice kt+1 (into the other register set) and,
// every other one, with one of the 8 loads that refill stage kt % NS with
// slice kt + NS.  The pairs are pinned with sched_barrier.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm_lines.hpp"
#include "gemm.h"

namespace gemm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int fp8_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int kn_swz(int k) { return 2 * (k & 7); }
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

template <int NS, int GROUP_M, int OUT, bool AKN = false, bool BKN = false>
__global__ void __launch_bounds__(256)
fp8_ring_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint8_t>(p);
    static_assert(NS == 4, "the stage arrays and the register-set parity assume four stages");
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int kA = BM * BK;          // 16 KB of A per slice
    constexpr int kB = BN * BK;          // 16 KB of B per slice
    constexpr int kStage = kA + kB;
    __shared__ __attribute__((aligned(1024))) char st0[kStage], st1[kStage], st2[kStage], st3[kStage];
    auto stage_base = [&](int st) -> char * { return st == 0 ? st0 : st == 1 ? st1 : st == 2 ? st2 : st3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // Load instruction j (0..3) of this wave fills 1 KB block 4*wave + j of a
    // panel: rows 16*blk .. +15, lane -> row 16*blk + lane/4, physical chunk
    // lane%4, which holds logical chunk (lane%4) ^ swizzle(row).
    // For a K x (M or N) panel, instruction j fills k rows 4*(4*wave + j) ..
    // +3: lane -> row 4*(4*wave + j) + lane/16, physical chunk lane%16, which
    // holds logical chunk (lane%16) ^ kn_swz(row).
    uint32_t goff_a[4], goff_b[4];
    int kc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 16 * (4 * wave + j) + (lane >> 2);
        const int lc = (lane & 3) ^ fp8_swz(row);
        kc[j] = 16 * lc;
        const int kr = 4 * (4 * wave + j) + (lane >> 4);
        const int cc = (lane & 15) ^ kn_swz(kr);
        goff_a[j] = AKN ? (uint32_t)(kr * lda + 16 * cc) : panel_off(row, a_rows, lda, 16 * lc, 1);
        goff_b[j] = BKN ? (uint32_t)(kr * ldb + 16 * cc) : panel_off(row, b_rows, ldb, 16 * lc, 1);
    }
    // Resources of slice kt, rebased per slice.  Slices past K fall outside
    // the extents, rows past M (or N) read the last valid row, and a chunk at
    // or past K in a row gets 2^31 added to its offset.
    // A K x (M or N) panel's extent ends at its last k row; rows past K and
    // the last row's columns past M (N) read as zero.
    auto slice_rsrc = [&](int kt, rsrc_t &ra, rsrc_t &rb) {
        const int k0 = kt * BK;
        if (AKN)
            ra = make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent((int64_t)(K - k0 - 1) * lda + (M - m0)));
        else
            ra = make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent((int64_t)(a_rows - 1) * lda + (K - k0)));
        if (BKN)
            rb = make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent((int64_t)(K - k0 - 1) * ldb + (N - n0)));
        else
            rb = make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent((int64_t)(b_rows - 1) * ldb + (K - k0)));
    };
    // Load instruction j (0..7) of slice kt into `stage`: j < 4 fills A block
    // 4*wave + j, j >= 4 fills B block 4*wave + j - 4.
    auto dma = [&](int kt, int stage, const rsrc_t &ra, const rsrc_t &rb, int j) {
        const int jj = j & 3;
        const bool kn = j < 4 ? AKN : BKN;     // k rows past K already fall outside the extent
        const uint32_t poison = kn ? 0u : (uint32_t)(kc[jj] >= K - kt * BK) << 31;
        char *dst = stage_base(stage) + (j < 4 ? 0 : kA) + (4 * wave + jj) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 4 ? ra : rb, (lds_void *)dst, 16,
                                                 (j < 4 ? goff_a[jj] : goff_b[jj]) + poison, 0, 0, 0);
    };
    // Fragment reads: lane (h, l32) of fragment f reads row 32*f + l32 of the
    // wave's 128-row block, logical chunks 2h and 2h+1.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int sw = fp8_swz(l32);
    const uint32_t ch0 = 16 * ((2 * h) ^ sw), ch1 = 16 * ((2 * h + 1) ^ sw);
    const uint32_t fa_row = (uint32_t)((wm * 128 + l32) * BK);
    const uint32_t fb_row = (uint32_t)(kA + (wn * 128 + l32) * BK);

    // Transposing reads of a K x (M or N) panel: lane s of each 16-lane group
    // points at k row 32h + 8q + e(s) and the half 8*(s%2) of the 16-byte
    // chunk holding the group's 16 columns.
    const int s16 = lane & 15;
    const int e_src = ((s16 >> 1) & 3) + 4 * (s16 >> 3);
    auto kn_off = [&](uint32_t region, int wcol, int f, int q) -> uint32_t {
        const int kr = 32 * h + 8 * q + e_src;
        const int c = wcol / 16 + 2 * f + (l32 >> 4);
        return region + (uint32_t)(kr * 256 + 16 * (c ^ kn_swz(kr)) + 8 * (s16 & 1));
    };

    i32x8 fa[2][4], fb[2][4];
    // Read r of the slice in `stage` into register set `set`: the first NRA
    // are A's (two 16-byte halves, or four transposing 8-byte reads, per
    // fragment), then B's.
    constexpr int NRA = AKN ? 16 : 8, NRB = BKN ? 16 : 8, NR = NRA + NRB;
    auto read_slot = [&](int stage, int set, int r) {
        const char *base = stage_base(stage);
        const bool is_a = r < NRA;
        const bool kn = is_a ? AKN : BKN;
        const int rr = is_a ? r : r - NRA;
        i32x8 *frags = is_a ? fa[set] : fb[set];
        if (kn) {
            const int f = rr >> 2, q = rr & 3;
            const uint32_t off = is_a ? kn_off(0, wm * 128, f, q) : kn_off(kA, wn * 128, f, q);
            const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(base + off));
            frags[f][2 * q] = v[0];
            frags[f][2 * q + 1] = v[1];
        } else {
            const int f = (rr >> 1) & 3;
            const uint32_t off = (is_a ? fa_row : fb_row) + 32 * BK * f + ((rr & 1) ? ch1 : ch0);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(base + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) frags[f][4 * (rr & 1) + e] = (int)v[e];
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // B^T as the first operand and A^T as the second, as in the bf16 ring:
    // each lane then holds runs of 4 consecutive columns of one row of C.
    auto mma = [&](int set, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0, 0,
                                                                     0, 0);
    };

    const int nk = (K + BK - 1) / BK;
    {
        rsrc_t ra, rb;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            slice_rsrc(st, ra, rb);
#pragma unroll
            for (int j = 0; j < 8; ++j) dma(st, st, ra, rb, j);
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 * (NS - 1)));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_slot(0, 0, r);
    for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int kt = kb + u;
            // This wave's reads of slice kt are done and slice kt+1 has
            // landed; after the barrier, for every wave.
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 * (NS - 2)));
            __builtin_amdgcn_s_barrier();
            rsrc_t ra, rb;
            slice_rsrc(kt + NS, ra, rb);      // zeros past the end
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(u & 1, t);
#pragma unroll
                for (int r = t * NR / 16; r < (t + 1) * NR / 16; ++r) read_slot((u + 1) % NS, (u + 1) & 1, r);
                if ((t & 1) == 0) dma(kt + NS, u, ra, rb, t >> 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Epilogue.  Register 4g + t of lane (h, l32) in fragment (fm, fn) is
    // C[row m0 + wm*128 + 32*fm + l32][column n0 + wn*128 + 32*fn + 8*g + 4*h + t].
    // A run of 4 columns may straddle N (no constraint on N here): such runs,
    // and C without 16-byte alignment, take element accesses.  The activation
    // is a uniform branch per run of 4 values, taken on values already moved
    // out of the accumulators: with one branch around the whole tile the
    // compiler copied every accumulator to an architectural register at the
    // branch and had to put some in scratch memory.
    const float alpha = p.alpha, beta = p.beta;
    const bool vec_c = ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 4 == 0);
    {
        const bool vec_o = out_vec4<OUT>(p);
        const int act = p.act;
        // fp32 output without C0 or an activation: each group of four runs
        // takes one branch-free path (a branch per run on beta and the
        // activation cost 3.5% of the 8192^3 call).  The quantising outputs
        // keep the single loop: a second copy of their conversions pushed
        // the accumulators to scratch.
        const bool plain = OUT == GEMM_OUT_F32 && beta == 0.0f && act == GEMM_ACT_NONE;
#pragma unroll
            for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * 128 + 32 * fn + 8 * g + 4 * h;
                    if (col >= N) continue;
                    const bool whole = col + 4 <= N;
                    float b[4];   // -0.0 is the identity of IEEE addition, signed zeros included
#pragma unroll
                    for (int t = 0; t < 4; ++t) b[t] = (p.bias != nullptr && col + t < N) ? p.bias[col + t] : -0.0f;
                    if (OUT == GEMM_OUT_F32 && plain) {
#pragma unroll
                        for (int fm = 0; fm < 4; ++fm) {
                            const int row = m0 + wm * 128 + 32 * fm + l32;
                            if (row >= M) continue;
                            f32x4 v;
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = alpha * acc[fm][fn][4 * g + t] + b[t];
                            if (whole)
                                store_out4<OUT>(p, row, col, v, vec_o);
                            else
                                store_out_first<OUT>(p, row, col, v, N - col);
                        }
                        continue;
                    }
#pragma unroll
                    for (int fm = 0; fm < 4; ++fm) {
                        const int row = m0 + wm * 128 + 32 * fm + l32;
                        if (row >= M) continue;
                        const float *cp = p.C + (int64_t)row * p.ldc + col;
                        f32x4 v = {alpha * acc[fm][fn][4 * g], alpha * acc[fm][fn][4 * g + 1],
                                   alpha * acc[fm][fn][4 * g + 2], alpha * acc[fm][fn][4 * g + 3]};
                        if (beta != 0.0f) {
                            f32x4 c0;
                            if (whole && vec_c) {
                                c0 = *reinterpret_cast<const f32x4 *>(cp);
                            } else {
#pragma unroll
                                for (int t = 0; t < 4; ++t) c0[t] = col + t < N ? cp[t] : 0.0f;
                            }
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = fmaf(beta, c0[t], v[t]);
                        }
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] += b[t];
                        if (act == GEMM_ACT_GELU) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = ActGelu::apply(v[t]);
                        } else if (act == GEMM_ACT_RELU) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = ActRelu::apply(v[t]);
                        }
                        if (whole)
                            store_out4<OUT>(p, row, col, v, vec_o);
                        else
                            store_out_first<OUT>(p, row, col, v, N - col);
                    }
                }
            }
    }
}

template <int NS, int GROUP_M, bool AKN = false, bool BKN = false>
hipError_t launch_fp8_ring(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn =
        out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&fp8_ring_kernel<NS, GROUP_M, GEMM_OUT_BF16, AKN, BKN>)
        : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&fp8_ring_kernel<NS, GROUP_M, GEMM_OUT_FP8, AKN, BKN>)
                              : reinterpret_cast<const void *>(&fp8_ring_kernel<NS, GROUP_M, GEMM_OUT_F32, AKN, BKN>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

// The same ring at 128 x 128 (each wave 64 x 64, 2 x 2 fragments), for the
// layouts without a 128 x 128 whole-line kernel: four 16 KB stages (two
// workgroups per compute unit), per slice 4 matrix instructions per wave,
// each paired with a quarter of the next slice's fragment reads and one of
// the slice's 4 loads.  A K x (M or N) slice is [64 k rows][128 columns];
// its 16-byte chunk c of row k sits at c ^ (k % 8), which gives the eight
// rows of a transposing read eight different chunk columns.  Byte pairing,
// slice order and the extra zero slices past K are the 256 x 256 ring's, so
// the two give the same bits.  The epilogue is the whole-line kernels'.
template <int OUT, bool AKN, bool BKN>
__global__ void __launch_bounds__(256)
fp8_ring128_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint8_t>(p);
    constexpr int NS = 4, BM = 128, BN = 128, BK = 64;
    constexpr int kA = BM * BK;          // 8 KB of A per slice
    constexpr int kB = BN * BK;          // 8 KB of B per slice
    constexpr int kStage = kA + kB;
    __shared__ __attribute__((aligned(1024))) char st0[kStage], st1[kStage], st2[kStage], st3[kStage];
    auto stage_base = [&](int st) -> char * { return st == 0 ? st0 : st == 1 ? st1 : st == 2 ? st2 : st3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // Load j (0..1) of this wave fills 1 KB block i = 2*wave + j of a panel:
    // k-contiguous, rows 16i .. +15 (lane -> row 16i + lane/4, physical chunk
    // lane%4 holding logical chunk (lane%4) ^ swizzle(row)); K x (M or N), k
    // rows 8i .. 8i+7 (lane -> k row 8i + lane/8, physical chunk lane%8
    // holding logical chunk (lane%8) ^ (k % 8)).
    uint32_t goff_a[2], goff_b[2];
    int kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = 2 * wave + j;
        const int row = 16 * i + (lane >> 2);
        const int lc = (lane & 3) ^ fp8_swz(row);
        kc[j] = 16 * lc;
        const int kr = 8 * i + (lane >> 3);
        const int cc = (lane & 7) ^ (kr & 7);
        goff_a[j] = AKN ? (uint32_t)(kr * lda + 16 * cc) : panel_off(row, a_rows, lda, 16 * lc, 1);
        goff_b[j] = BKN ? (uint32_t)(kr * ldb + 16 * cc) : panel_off(row, b_rows, ldb, 16 * lc, 1);
    }
    // Resources of slice kt, rebased per slice, as in the 256 x 256 ring.
    auto slice_rsrc = [&](int kt, rsrc_t &ra, rsrc_t &rb) {
        const int k0 = kt * BK;
        if (AKN)
            ra = make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent((int64_t)(K - k0 - 1) * lda + (M - m0)));
        else
            ra = make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent((int64_t)(a_rows - 1) * lda + (K - k0)));
        if (BKN)
            rb = make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent((int64_t)(K - k0 - 1) * ldb + (N - n0)));
        else
            rb = make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent((int64_t)(b_rows - 1) * ldb + (K - k0)));
    };
    // Load j (0..3) of slice kt into `stage`: j < 2 fills A block 2*wave + j,
    // j >= 2 B block 2*wave + j - 2.
    auto dma = [&](int kt, int stage, const rsrc_t &ra, const rsrc_t &rb, int j) {
        const int jj = j & 1;
        const bool kn = j < 2 ? AKN : BKN;     // k rows past K already fall outside the extent
        const uint32_t poison = kn ? 0u : (uint32_t)(kc[jj] >= K - kt * BK) << 31;
        char *dst = stage_base(stage) + (j < 2 ? 0 : kA) + (2 * wave + jj) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 2 ? ra : rb, (lds_void *)dst, 16,
                                                 (j < 2 ? goff_a[jj] : goff_b[jj]) + poison, 0, 0, 0);
    };
    // Fragment reads: lane (h, l32) of fragment f reads row 32*f + l32 of the
    // wave's 64-row block, logical chunks 2h and 2h+1 (k-contiguous); with a
    // K x (M or N) panel, lane s of each 16-lane group points at k row 32h +
    // 8q + e(s) and the half 8*(s%2) of the chunk holding the group's 16
    // columns (the 256 x 256 ring's transposing reads on 128-byte rows).
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int sw = fp8_swz(l32);
    const uint32_t ch0 = 16 * ((2 * h) ^ sw), ch1 = 16 * ((2 * h + 1) ^ sw);
    const uint32_t fa_row = (uint32_t)((wm * 64 + l32) * BK);
    const uint32_t fb_row = (uint32_t)(kA + (wn * 64 + l32) * BK);
    const int s16 = lane & 15;
    const int e_src = ((s16 >> 1) & 3) + 4 * (s16 >> 3);
    auto kn_off = [&](uint32_t region, int wcol, int f, int q) -> uint32_t {
        const int kr = 32 * h + 8 * q + e_src;
        const int c = wcol / 16 + 2 * f + (l32 >> 4);
        return region + (uint32_t)(kr * 128 + 16 * (c ^ (kr & 7)) + 8 * (s16 & 1));
    };

    i32x8 fa[2][2], fb[2][2];
    constexpr int NRA = AKN ? 8 : 4, NRB = BKN ? 8 : 4, NR = NRA + NRB;
    auto read_slot = [&](int stage, int set, int r) {
        const char *base = stage_base(stage);
        const bool is_a = r < NRA;
        const bool kn = is_a ? AKN : BKN;
        const int rr = is_a ? r : r - NRA;
        i32x8 *frags = is_a ? fa[set] : fb[set];
        if (kn) {
            const int f = rr >> 2, q = rr & 3;
            const uint32_t off = is_a ? kn_off(0, wm * 64, f, q) : kn_off(kA, wn * 64, f, q);
            const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(base + off));
            frags[f][2 * q] = v[0];
            frags[f][2 * q + 1] = v[1];
        } else {
            const int f = (rr >> 1) & 1;
            const uint32_t off = (is_a ? fa_row : fb_row) + 32 * BK * f + ((rr & 1) ? ch1 : ch0);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(base + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) frags[f][4 * (rr & 1) + e] = (int)v[e];
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto mma = [&](int set, int t) {
        const int i = t >> 1, j = t & 1;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0, 0,
                                                                     0, 0);
    };

    const int nk = (K + BK - 1) / BK;
    {
        rsrc_t ra, rb;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            slice_rsrc(st, ra, rb);
#pragma unroll
            for (int j = 0; j < 4; ++j) dma(st, st, ra, rb, j);
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * (NS - 1)));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_slot(0, 0, r);
    for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int kt = kb + u;
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * (NS - 2)));
            __builtin_amdgcn_s_barrier();
            rsrc_t ra, rb;
            slice_rsrc(kt + NS, ra, rb);      // zeros past the end
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                mma(u & 1, t);
#pragma unroll
                for (int r = t * NR / 4; r < (t + 1) * NR / 4; ++r) read_slot((u + 1) % NS, (u + 1) & 1, r);
                dma(kt + NS, u, ra, rb, t);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // Every load has landed and every wave is done with the stages before the
    // epilogue reuses them: 16 KB of staging per wave, stage `wave`.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    char *stg = stage_base(wave);
    lines_epilogue<OUT, true>(p, acc, [&](int row) -> char * { return stg + row * 256; }, m0, n0, wm, wn, lane);
}

template <bool AKN, bool BKN>
hipError_t launch_fp8_ring128(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 127) / 128, tiles_n = (p.N + 127) / 128;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&fp8_ring128_kernel<GEMM_OUT_BF16, AKN, BKN>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&fp8_ring128_kernel<GEMM_OUT_FP8, AKN, BKN>)
                                           : reinterpret_cast<const void *>(&fp8_ring128_kernel<GEMM_OUT_F32, AKN, BKN>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

#define FP8_RING_INSTANCES(AKN, BKN)                                                             \
    template __global__ void fp8_ring_kernel<4, 4, GEMM_OUT_F32, AKN, BKN>(GemmParams, int, int);  \
    template __global__ void fp8_ring_kernel<4, 4, GEMM_OUT_BF16, AKN, BKN>(GemmParams, int, int); \
    template __global__ void fp8_ring_kernel<4, 4, GEMM_OUT_FP8, AKN, BKN>(GemmParams, int, int);
FP8_RING_INSTANCES(false, false)
FP8_RING_INSTANCES(false, true)
FP8_RING_INSTANCES(true, true)
FP8_RING_INSTANCES(true, false)
template __global__ void fp8_ring128_kernel<GEMM_OUT_F32, false, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_BF16, false, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_FP8, false, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_F32, true, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_BF16, true, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_FP8, true, true>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_F32, true, false>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_BF16, true, false>(GemmParams, int, int);
template __global__ void fp8_ring128_kernel<GEMM_OUT_FP8, true, false>(GemmParams, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// vec_a = vec_b = 16: A, B, lda, ldb and K multiples of 16 bytes.
const KernelDesc kFp8TiledKernels[] = {
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 256, 256, 64, 256, 16, 16, "fp8_mfma32_256x256x64_w2x2_nt_ring4",
     &launch_fp8_ring<4, 4>, 0, nullptr, kLayoutNT, false, kOutAll},
    // A or B stored the other way (K x M, K x N): its rows, M or N long, are
    // whole 16-byte chunks too.
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 256, 256, 64, 256, 16, 16, "fp8_mfma32_256x256x64_w2x2_nn_ring4",
     &launch_fp8_ring<4, 4, false, true>, 0, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 256, 256, 64, 256, 16, 16, "fp8_mfma32_256x256x64_w2x2_tn_ring4",
     &launch_fp8_ring<4, 4, true, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 256, 256, 64, 256, 16, 16, "fp8_mfma32_256x256x64_w2x2_tt_ring4",
     &launch_fp8_ring<4, 4, true, false>, 0, nullptr, kLayoutTT, false, kOutAll},
    // 128 x 128 for the layouts without a whole-line kernel of that tile.
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 128, 128, 64, 256, 16, 16, "fp8_mfma32_128x128x64_w2x2_nn_ring4",
     &launch_fp8_ring128<false, true>, 0, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 128, 128, 64, 256, 16, 16, "fp8_mfma32_128x128x64_w2x2_tn_ring4",
     &launch_fp8_ring128<true, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 128, 128, 64, 256, 16, 16, "fp8_mfma32_128x128x64_w2x2_tt_ring4",
     &launch_fp8_ring128<true, false>, 0, nullptr, kLayoutTT, false, kOutAll},
};
const int kFp8TiledKernelCount = sizeof(kFp8TiledKernels) / sizeof(kFp8TiledKernels[0]);
#endif

}  // namespace gemm
