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
    apply_k_split<float>(p);
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

    // A row panel: its extent ends right after the last valid element (the
    // host keeps it below 2^31 bytes); rows at or past M read row M - 1.
    const float *a_panel = static_cast<const float *>(p.A) + (int64_t)m0 * lda;
    const int a_rows = min(BM, M - m0);
    const rsrc_t ra = make_rsrc(a_panel, clamp_extent(((int64_t)(a_rows - 1) * lda + K) * 4));

    uint32_t a_off[Cfg::kAPer];
    int a_k[Cfg::kAPer], a_lds[Cfg::kAPer];
#pragma unroll
    for (int i = 0; i < Cfg::kAPer; ++i) {
        const int c = tid + i * Cfg::kThreads;
        const int r = c / (BK / VA), kc = (c % (BK / VA)) * VA;
        a_off[i] = panel_off(r, a_rows, lda, kc, 4);
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
                    float v = alpha * acc[fm][fn][r];
                    if constexpr (quantising_epilogue(Cfg::kWaveM * Cfg::kWaveN / 64)) {
                        if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)row * p.ldc + col], v);
                        store_out_any(p, row, col, epilogue_value(v, col, p.bias, p.act));
                    } else {
                        float *cp = p.C + (int64_t)row * p.ldc + col;
                        if (beta != 0.0f) v = fmaf(beta, *cp, v);
                        *cp = epilogue_value(v, col, p.bias, p.act);
                    }
                }
            }
        }
    }
}

// Ring form for 16-byte-aligned operands: the 256 x 256 tile, 16-deep k
// slices and 4 waves of the kernel above, with three changes that remove its
// stalls (each slice is 128 matrix instructions per wave, so a few hundred
// idle cycles per slice are several percent):
//   * Panels go straight from HBM into an LDS ring of NS slices with
//     buffer_load ... lds (lane i of a wave instruction lands at the LDS base
//     + 16*i), so no registers stage them and no LDS stores are issued.  Slice
//     kt+NS is requested as soon as slice kt has been consumed ("What is
//     left": asynchronous copies and multi-buffering).
//       A slice: [256 rows][4 chunks of 16 B] (k contiguous), chunk ^= (row >> 2) & 3;
//       B slice: [16 k rows][256 columns], as in HBM.
//   * Column j of the wave's 32 x 32 fragment fn stands for column 4*j + fn
//     of its 128-column block, so a lane's four B values of a k pair are
//     four consecutive floats (one 16-byte read) and its results for a row
//     are four consecutive columns of C (one 16-byte store).
//   * Each slice is 8 steps of 16 MFMAs (one k pair per step).  The B values
//     of step s+1 are read during step s; after step 5 every wave waits for
//     slice kt+1 to land and for the reads of this stage to finish
//     (barrier), then steps 6 and 7 run while the stage is refilled and the
//     next slice's A fragments and first B values are read.  The other
//     instructions are pinned between MFMAs with sched_barrier.
// Loads complete in issue order: before the barrier of slice kt the only
// loads allowed in flight are the 8*(NS-2) of the slices after kt+1.
//
// BT: B is stored N x K (k contiguous along each of its rows), the shape of
// A.  Its slices then take A's layout, loads and fragment reads (k chunks
// past K masked the same way), and B's fragment goes in as the matrix
// instruction's first operand: lane (h, l32) of fragment (fm, fn) then holds
// runs of 4 consecutive columns of one row of C, as in the bf16 ring.  N is
// free; runs of columns that straddle N are stored element by element.
//
// AT: A is stored K x M (m contiguous), the shape of an untransposed B, so
// its slices take B's layout and loads ([16 k rows][256 m]), and a lane's
// 16-byte read at row k gives it one value for each of its four A
// fragments: row i of fragment fm stands for m = 4*i + fm of the wave's
// 128-row block, as column j of fragment fn stands for n = 4*j + fn.  Only
// the rows of C the epilogue addresses change.
template <int NS, int GROUP_M, int OUT, bool BT, bool AT = false>
__global__ void __launch_bounds__(256)
f32_ring_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<float>(p);
    static_assert(NS % 2 == 0, "the two A-fragment register sets alternate with the stage");
    constexpr int BM = 256, BN = 256, BK = 16, kSteps = 8;
    constexpr int kA = BM * BK * 4;     // 16 KB of A per slice
    constexpr int kB = BK * BN * 4;     // 16 KB of B per slice
    constexpr int kStage = kA + kB;
    // One array per stage: with distinct objects the compiler can tell that
    // fragment reads of one stage do not depend on loads still landing in
    // another.
    __shared__ __attribute__((aligned(1024))) char st0[kStage], st1[kStage], st2[kStage], st3[kStage];
    auto stage_base = [&](int st) -> char * { return st == 0 ? st0 : st == 1 ? st1 : st == 2 ? st2 : st3; };
    static_assert(NS <= 4, "four stage arrays");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const float *A = static_cast<const float *>(p.A);
    const float *B = static_cast<const float *>(p.B);
    const int a_rows = min(BM, M - m0);
    const int b_rows = min(BN, N - n0);     // rows of a B^T slice (BT)

    // Load instruction j of this wave: j < 4 fills A block 4*wave + j (rows
    // 16*blk .. +15; lane -> row 16*blk + lane/4, physical chunk lane%4);
    // j >= 4 fills B row 4*wave + j - 4 (lane -> columns 4*lane .. +3), or
    // with BT block 4*wave + j - 4 of B^T exactly as for A.
    uint32_t a_goff[4], b_goff[4];
    int a_kc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 16 * (4 * wave + j) + (lane >> 2);
        const int lc = (lane & 3) ^ ((row >> 2) & 3);
        a_kc[j] = 4 * lc;
        a_goff[j] = AT ? (uint32_t)((4 * wave + j) * lda + 4 * lane) * 4u : panel_off(row, a_rows, lda, 4 * lc, 4);
        b_goff[j] = BT ? panel_off(row, b_rows, ldb, 4 * lc, 4) : (uint32_t)((4 * wave + j) * ldb + 4 * lane) * 4u;
    }
    // Resources of slice kt, rebased per slice: k rows past K fall outside the
    // extents, rows past M (past N for B^T) read the last valid row, and a
    // chunk at or past K in a row of A (or B^T) gets 2^31 added to its offset.
    auto slice_rsrc = [&](int kt, rsrc_t &ra, rsrc_t &rb) {
        const int k0 = kt * BK;
        if (AT)
            ra = make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent(((int64_t)(K - k0 - 1) * lda + (M - m0)) * 4));
        else
            ra = make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 4));
        if (BT)
            rb = make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent(((int64_t)(b_rows - 1) * ldb + (K - k0)) * 4));
        else
            rb = make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 4));
    };
    auto dma = [&](int kt, int stage, const rsrc_t &ra, const rsrc_t &rb, int j) {
        const int jj = j & 3;
        const uint32_t poison = (uint32_t)(a_kc[jj] >= K - kt * BK) << 31;
        if (j < 4) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(stage_base(stage) + (4 * wave + j) * 1024), 16,
                                                     a_goff[j] + (AT ? 0u : poison), 0, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(stage_base(stage) + kA + (4 * wave + jj) * 1024),
                                                     16, b_goff[jj] + (BT ? poison : 0u), 0, 0, 0);
        }
    };

    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    // A fragment (fm, q): row wm*128 + 32*fm + l32, k = 8h + 4q .. +3.
    // B values of step s: row 8h + s, columns wn*128 + 4*l32 .. +3.
    uint32_t fa_off[2], fbt_off[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        fa_off[q] = (uint32_t)((wm * 128 + l32) * 64 + 16 * ((2 * h + q) ^ ((l32 >> 2) & 3)));
        fbt_off[q] = (uint32_t)(kA + (wn * 128 + l32) * 64 + 16 * ((2 * h + q) ^ ((l32 >> 2) & 3)));
    }
    const uint32_t fb_off = (uint32_t)(kA + 8 * h * 1024 + (wn * 128 + 4 * l32) * 4);
    const uint32_t fat_off = (uint32_t)(8 * h * 1024 + (wm * 128 + 4 * l32) * 4);   // A^T values (AT)

    f32x4 af[2][4][2];
    f32x4 bv[kSteps];
    f32x4 bf[BT ? 2 : 1][4][2];    // B^T fragments, like af (BT only)
    f32x4 av[kSteps];              // A^T values of each step, like bv (AT only)
    auto read_a = [&](int stage, int set, int fm) {
        if constexpr (!AT) {
            const char *base = stage_base(stage);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                af[set][fm][q] = *reinterpret_cast<const f32x4 *>(base + fa_off[q] + 2048 * fm);
        }
    };
    auto read_at = [&](int stage, int s) {
        if constexpr (AT) av[s] = *reinterpret_cast<const f32x4 *>(stage_base(stage) + fat_off + 1024 * s);
    };
    auto read_b = [&](int stage, int s) {
        if constexpr (!BT) bv[s] = *reinterpret_cast<const f32x4 *>(stage_base(stage) + fb_off + 1024 * s);
    };
    auto read_bt = [&](int stage, int set, int fn) {
        if constexpr (BT) {
            const char *base = stage_base(stage);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                bf[set][fn][q] = *reinterpret_cast<const f32x4 *>(base + fbt_off[q] + 2048 * fn);
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // MFMA t (0..15) of step s: fragment (t/4, t%4); lane half h supplies
    // k = s (h = 0) or 8 + s (h = 1) of the slice for both operands.
    auto mma = [&](int set, int s, int t) {
        const int fm = t >> 2, fn = t & 3;
        const float a = AT ? av[s][fm] : af[set][fm][s >> 2][s & 3];
        if constexpr (BT)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[set][fn][s >> 2][s & 3], a, acc[fm][fn], 0, 0, 0);
        else
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv[s][fn], acc[fm][fn], 0, 0, 0);
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
    for (int fm = 0; fm < 4; ++fm) read_a(0, 0, fm);
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) read_bt(0, 0, fn);
    read_b(0, 0);
    read_at(0, 0);
    for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int kt = kb + u, set = u & 1, nxt = (u + 1) % NS;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 6; ++s) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    mma(set, s, t);
                    if (t == 0) read_b(u, s + 1);
                    if (t == 2) read_at(u, s + 1);
                    if (s == 5 && t == 1) read_b(u, 7);
                    if (s == 5 && t == 3) read_at(u, 7);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 * (NS - 2)));
            __builtin_amdgcn_s_barrier();
            rsrc_t ra, rb;
            slice_rsrc(kt + NS, ra, rb);     // zeros past the end
            __builtin_amdgcn_sched_barrier(0);
            // Steps 6 and 7 with 8 loads and 5 fragment reads between them.
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                mma(set, 6 + (q >> 4), q & 15);
                if ((q & 1) == 0 && q < 16) dma(kt + NS, u, ra, rb, q >> 1);
                if ((q & 1) == 1 && q < 8) read_a(nxt, set ^ 1, q >> 1);
                if (BT && (q & 1) == 1 && q >= 9 && q < 16) read_bt(nxt, set ^ 1, (q - 9) >> 1);
                if (q == 9) read_b(nxt, 0);
                if (q == 11) read_at(nxt, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Epilogue.  Register r of lane (h, l32) in fragment (fm, fn) is row
    // 32*fm + 8*(r/4) + 4*h + r%4 of the wave tile, column 4*l32 + fn; N is a
    // multiple of 4 on this path, so each run of 4 columns is wholly inside
    // or outside C.  The branch on the activation is taken once for the whole
    // tile, so each case is one fully unrolled pass and the accumulators stay
    // in registers.
    const float alpha = p.alpha, beta = p.beta;
    const bool vec_c = ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 4 == 0);
    if constexpr (BT) {
        // B^T was the first operand: register 4g + t of lane (h, l32) in
        // fragment (fm, fn) is C[row m0 + wm*128 + 32*fm + l32 (with A^T:
        // 4*l32 + fm)][column n0 + wn*128 + 32*fn + 8*g + 4*h + t].
        with_activation(p.act, [&](auto act) {
            using Act = decltype(act);
            const bool vec_o = out_vec4<OUT>(p);
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
#pragma unroll
                    for (int fm = 0; fm < 4; ++fm) {
                        const int row = AT ? m0 + wm * 128 + 4 * l32 + fm : m0 + wm * 128 + 32 * fm + l32;
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
                        for (int t = 0; t < 4; ++t) v[t] = Act::apply(v[t] + b[t]);
                        if (whole)
                            store_out4<OUT>(p, row, col, v, vec_o);
                        else
                            store_out_first<OUT>(p, row, col, v, N - col);
                    }
                }
            }
        });
        return;
    }
    const int col = n0 + wn * 128 + 4 * l32;
    if (col >= N) return;
    float b[4];   // -0.0 is the identity of IEEE addition, signed zeros included
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = p.bias != nullptr ? p.bias[col + e] : -0.0f;
    with_activation(p.act, [&](auto act) {
        using Act = decltype(act);
        const bool vec_o = out_vec4<OUT>(p);
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 8 * (r >> 2) + 4 * h + (r & 3);     // row of the fragment
                    const int row = AT ? m0 + wm * 128 + 4 * i + fm : m0 + wm * 128 + 32 * fm + i;
                    if (row >= M) continue;
                    f32x4 v = {alpha * acc[fm][0][r], alpha * acc[fm][1][r], alpha * acc[fm][2][r],
                               alpha * acc[fm][3][r]};
                    if (beta != 0.0f) {
                        const float *cp = p.C + (int64_t)row * p.ldc + col;
                        const f32x4 c0 =
                            vec_c ? *reinterpret_cast<const f32x4 *>(cp) : f32x4{cp[0], cp[1], cp[2], cp[3]};
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = fmaf(beta, c0[e], v[e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = Act::apply(v[e] + b[e]);
                    store_out4<OUT>(p, row, col, v, vec_o);
                }
            }
    });
}

template <int NS, int GROUP_M, bool BT = false, bool AT = false>
hipError_t launch_f32_ring(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn =
        out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&f32_ring_kernel<NS, GROUP_M, GEMM_OUT_BF16, BT, AT>)
        : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&f32_ring_kernel<NS, GROUP_M, GEMM_OUT_FP8, BT, AT>)
                              : reinterpret_cast<const void *>(&f32_ring_kernel<NS, GROUP_M, GEMM_OUT_F32, BT, AT>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

// 64 x 64 (F = 1) and 128 x 128 (F = 2) tiles on a direct-to-LDS ring of NS
// stages, each of the 4 waves owning F x F fragments of 32 x 32.  The
// register-staged kernel above holds one slice in flight, so every 16-deep
// slice waits out a whole global-load latency; here slice kt + NS - 1 is
// requested as slice kt starts ("A GEMM Kernel, Step by Step", "What is
// left": asynchronous copies and multi-buffering).  64 x 64: six stages of
// 8 KB, three workgroups per compute unit; 128 x 128: four of 16 KB, two.
//   A slice: [BM rows][4 chunks of 16 B] (k contiguous), logical chunk c of
//     row r at c ^ ((r >> 2) & 3), as in the 256 x 256 ring.  VA = 4: 16-byte
//     loads (16 rows per wave instruction).  VA = 1 (rows of A not 16-byte
//     aligned, such as an odd K): 4-byte loads (4 rows per wave instruction),
//     lane i landing at 4i bytes, so each lane fetches the element that
//     belongs at its LDS position under the swizzle.
//   B slice: [16 k rows][BN columns] as in HBM, k rows 8 .. 15 starting 128
//     bytes later so that the two lane halves' reads (k rows s and 8 + s)
//     fall in different banks.
// BT (B stored N x K): B's slice takes A's layout and 16-byte loads, and its
// fragments are read as A's are; N is free.  AT (A stored K x M): A's slice
// takes B's layout and loads, and its values are read per step as B's are.
// Lane (h, l32) holds row l32 of each A fragment and column l32 of each B
// fragment at k = 8h + s for step s, so every accumulator sums k in the
// order of the kernel above, whatever the layout.
// A stage holds SUB 16-deep sub-slices, so one barrier serves 8*F*F*SUB
// matrix instructions.  Two (three stages of 16 KB for 64 x 64 tiles) were
// no faster than one; the table uses one, but the code shape with the
// per-sub-slice loop measured 4-12% faster on 64 x 64 tiles than the same
// kernel written without it (the compiler then starts the matrix
// instructions before the last fragment reads return).
template <int VA, int NS, int F, bool BT, bool AT, int SUB>
__global__ void __launch_bounds__(256)
f32_ring64_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<float>(p);
    static_assert(VA == 1 || VA == 4, "A loads of 4 or 16 bytes");
    static_assert(VA == 4 || !AT, "A stored K x M is loaded 16 bytes per lane");
    static_assert(NS >= 3 && NS <= 6, "six stage arrays");
    static_assert(F == 1 || F == 2, "64 x 64 or 128 x 128 tiles");
    static_assert(SUB == 1 || SUB == 2, "one or two 16-deep sub-slices per stage");
    constexpr int BM = 64 * F, BN = 64 * F, BK = 16;
    constexpr int kPad = 128;                    // k rows 8 .. 15 of a k-row slice start this much later
    constexpr int kRow = BN * 4;                 // bytes per k row of a k-row slice (BM == BN)
    constexpr int kKRowsPerLoad = 1024 / kRow;   // k rows per wave instruction of a k-row slice
    constexpr int kA = AT ? BK * kRow + kPad : BM * BK * 4;
    constexpr int kSub = kA + (BT ? BN * BK * 4 : BK * kRow + kPad);     // one 16-deep sub-slice
    constexpr int kStage = SUB * kSub;
    constexpr int kALoads = (VA == 4 || AT) ? F : 4 * F;     // A loads per wave per sub-slice
    constexpr int kLoads = SUB * (kALoads + F);
    __shared__ __attribute__((aligned(256))) char st0[kStage], st1[kStage], st2[kStage], st3[kStage], st4[kStage],
        st5[kStage];
    auto stage_base = [&](int st) -> char * {
        return st == 0 ? st0 : st == 1 ? st1 : st == 2 ? st2 : st == 3 ? st3 : st == 4 ? st4 : st5;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const float *A = static_cast<const float *>(p.A);
    const float *B = static_cast<const float *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // Loads of a k-contiguous slice (A, or B with BT): 16-byte instruction i
    // covers rows 16i .. +15 (lane -> row 16i + lane/4, physical chunk
    // lane%4) and lands at 1024 i; 4-byte instruction i covers rows 4i ..
    // 4i+3 (lane -> row 4i + lane/16, physical float lane%16) and lands at
    // 256 i.  Loads of a k-row slice (B, or A with AT): instruction i covers
    // k rows kKRowsPerLoad*i .. (lane -> k row kKRowsPerLoad*i + lane/(BN/4),
    // columns 4*(lane%(BN/4)) .. +3) and lands at 1024 i (+ kPad from k row
    // 8 on).  Load j of this wave is instruction kALoads*wave + j of A, F*wave
    // + j of B.
    // (Sized 8: hipcc's host pass rejects the LDS-load builtin when its offset
    // comes from an array whose size depends on a template parameter.)
    uint32_t a_goff[8], b_goff[2];
    int a_k[8], b_k[2];
    auto k_contig = [&](int i, int rows, int ld, bool narrow, uint32_t &goff, int &k) {
        int row;
        if (narrow) {
            row = 4 * i + (lane >> 4);
            const int pf = lane & 15;
            k = 4 * ((pf >> 2) ^ ((row >> 2) & 3)) + (pf & 3);
        } else {
            row = 16 * i + (lane >> 2);
            k = 4 * ((lane & 3) ^ ((row >> 2) & 3));
        }
        goff = panel_off(row, rows, ld, k, 4);
    };
    auto k_rows = [&](int i, int ld, uint32_t &goff) {
        const int krow = kKRowsPerLoad * i + lane / (BN / 4);
        goff = (uint32_t)(krow * ld + 4 * (lane % (BN / 4))) * 4u;
    };
    // LDS destinations of the loads (uniform across the wave).
    auto a_dst = [&](int j) {
        const int i = kALoads * wave + j;
        return AT ? 1024 * i + (kKRowsPerLoad * i >= 8 ? kPad : 0) : (VA == 4 ? 1024 * i : 256 * i);
    };
    auto b_dst = [&](int j) {
        const int i = F * wave + j;
        return kA + (BT ? 1024 * i : 1024 * i + (kKRowsPerLoad * i >= 8 ? kPad : 0));
    };
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
        a_k[j] = 0;
        if (AT)
            k_rows(kALoads * wave + j, lda, a_goff[j]);
        else
            k_contig(kALoads * wave + j, a_rows, lda, VA == 1, a_goff[j], a_k[j]);
    }
#pragma unroll
    for (int j = 0; j < F; ++j) {
        b_k[j] = 0;
        if (BT)
            k_contig(F * wave + j, b_rows, ldb, false, b_goff[j], b_k[j]);
        else
            k_rows(F * wave + j, ldb, b_goff[j]);
    }

    // Slice kt's loads into stage si, through resources rebased at the
    // slice: rows past M (N) read the last valid one, k past K gets 2^31
    // added to the offset (k-contiguous slices) or falls outside the extent
    // (k-row slices).
    auto issue_sub = [&](int ks, char *base) {
        const int k0 = BK * ks;
        const rsrc_t ra =
            AT ? make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent(((int64_t)(K - k0 - 1) * lda + (M - m0)) * 4))
               : make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 4));
        const rsrc_t rb =
            BT ? make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent(((int64_t)(b_rows - 1) * ldb + (K - k0)) * 4))
               : make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 4));
#pragma unroll
        for (int j = 0; j < kALoads; ++j) {
            const uint32_t poison = AT ? 0u : (uint32_t)(a_k[j] >= K - k0) << 31;
            if constexpr (VA == 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(base + a_dst(j)), 16, a_goff[j] + poison, 0,
                                                         0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(base + a_dst(j)), 4, a_goff[j] + poison, 0,
                                                         0, 0);
        }
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const uint32_t poison = BT ? (uint32_t)(b_k[j] >= K - k0) << 31 : 0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(base + b_dst(j)), 16, b_goff[j] + poison, 0, 0,
                                                     0);
        }
    };
    auto issue = [&](int kt, int si) {
#pragma unroll
        for (int t = 0; t < SUB; ++t) issue_sub(SUB * kt + t, stage_base(si) + kSub * t);
    };

    // Fragment reads: a k-contiguous fragment f of the wave's block is two
    // 16-byte reads (k = 8h .. 8h+7 of row l32); a k-row fragment gives one
    // float per step (k row 8h + s, column l32).
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    uint32_t fa_off[F][2], fbt_off[F][2];
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int chunk = 16 * ((2 * h + q) ^ ((l32 >> 2) & 3));
            fa_off[f][q] = (uint32_t)((wm * 32 * F + 32 * f + l32) * 64 + chunk);
            fbt_off[f][q] = (uint32_t)(kA + (wn * 32 * F + 32 * f + l32) * 64 + chunk);
        }
    const uint32_t arow_off = (uint32_t)(8 * h * kRow + (h ? kPad : 0) + (wm * 32 * F + l32) * 4);
    const uint32_t brow_off = (uint32_t)(kA + 8 * h * kRow + (h ? kPad : 0) + (wn * 32 * F + l32) * 4);
    f32x16 acc[F][F];
#pragma unroll
    for (int fm = 0; fm < F; ++fm)
#pragma unroll
        for (int fn = 0; fn < F; ++fn) acc[fm][fn] = f32x16{};

    // Slice kt: wait until it has landed (the loads of the NS - 2 slices after
    // it may still be in flight) and every wave has read the previous stage;
    // request slice kt + NS - 1 into that stage; multiply.
    auto slice = [&](int u, int kt) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kLoads * (NS - 2)));
        __builtin_amdgcn_s_barrier();
        issue(kt + NS - 1, (u + NS - 1) % NS);
#pragma unroll
        for (int t = 0; t < SUB; ++t) {
        const char *base = stage_base(u) + kSub * t;
        f32x4 a[F][2], b[F][2];
        float av[8][F], bv[8][F];
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (!AT) a[f][q] = *reinterpret_cast<const f32x4 *>(base + fa_off[f][q]);
                if (BT) b[f][q] = *reinterpret_cast<const f32x4 *>(base + fbt_off[f][q]);
            }
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
            for (int f = 0; f < F; ++f) {
                if (AT) av[st][f] = *reinterpret_cast<const float *>(base + arow_off + kRow * st + 128 * f);
                if (!BT) bv[st][f] = *reinterpret_cast<const float *>(base + brow_off + kRow * st + 128 * f);
            }
#pragma unroll
        for (int st = 0; st < 8; ++st)
#pragma unroll
            for (int fm = 0; fm < F; ++fm)
#pragma unroll
                for (int fn = 0; fn < F; ++fn) {
                    const float x = AT ? av[st][fm] : a[fm][st >> 2][st & 3];
                    const float y = BT ? b[fn][st >> 2][st & 3] : bv[st][fn];
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc[fm][fn], 0, 0, 0);
                }
        }
    };

    const int nk = (K + BK * SUB - 1) / (BK * SUB);
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st);
    const int nfull = nk / NS;
    int kb = 0;
    for (int it = 0; it < nfull; ++it, kb += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) slice(u, kb + u);
    }
    const int rem = nk - kb;
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (u < rem) slice(u, kb + u);
    // No load may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Register r of lane (h, l32) in fragment (fm, fn) is row 8*(r/4) + 4h +
    // r%4, column l32 of that fragment.
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int fn = 0; fn < F; ++fn) {
        const int col = n0 + wn * 32 * F + 32 * fn + l32;
        if (col >= N) continue;
#pragma unroll
        for (int fm = 0; fm < F; ++fm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * F + 32 * fm + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row >= M) continue;
                float v = alpha * acc[fm][fn][r];
                if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)row * p.ldc + col], v);
                store_out_any(p, row, col, epilogue_value(v, col, p.bias, p.act));
            }
        }
    }
}

template <int VA, int NS, int F, bool BT = false, bool AT = false, int SUB = 1>
hipError_t launch_f32_ring64(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 64 * F - 1) / (64 * F), tiles_n = (p.N + 64 * F - 1) / (64 * F);
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&f32_ring64_kernel<VA, NS, F, BT, AT, SUB>),
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
hipError_t launch_f32_tiled(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&f32_tiled_kernel<BM, BN, BK, WM, WN, VA, VB, GROUP_M>),
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(64 * WM * WN), argv, 0, stream);
}

#define F32_TILED(BM, BN, BK, WM, WN, VA, VB, G)                                              \
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, BM, BN, BK, 64 * WM * WN, VA, VB,                       \
     "f32_mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_a" #VA "b" #VB,                     \
     &launch_f32_tiled<BM, BN, BK, WM, WN, VA, VB, G>, 0, nullptr, kLayoutNN, false,                \
     quantising_epilogue((BM / WM) * (BN / WN) / 64) ? kOutAll : kOutF32}

// Explicit instantiations: the device pass never sees the host-only table
// below, so the kernels it needs are named here.
#define F32_RING_INSTANCES(BT, AT)                                                          \
    template __global__ void f32_ring_kernel<4, 4, GEMM_OUT_F32, BT, AT>(GemmParams, int, int);  \
    template __global__ void f32_ring_kernel<4, 4, GEMM_OUT_BF16, BT, AT>(GemmParams, int, int); \
    template __global__ void f32_ring_kernel<4, 4, GEMM_OUT_FP8, BT, AT>(GemmParams, int, int);
F32_RING_INSTANCES(false, false)
F32_RING_INSTANCES(true, false)
F32_RING_INSTANCES(false, true)
F32_RING_INSTANCES(true, true)
template __global__ void f32_ring64_kernel<4, 6, 1, false, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<1, 6, 1, false, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 6, 1, true, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 6, 1, false, true, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 6, 1, true, true, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 4, 2, false, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<1, 4, 2, false, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 4, 2, true, false, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 4, 2, false, true, 1>(GemmParams, int, int);
template __global__ void f32_ring64_kernel<4, 4, 2, true, true, 1>(GemmParams, int, int);
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
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 256, 256, 16, 256, 4, 4, "f32_mfma32_256x256x16_w2x2_a4b4_ring4",
     &launch_f32_ring<4, 4>, 0, nullptr, kLayoutNN, false, kOutAll},
    // B stored N x K: its rows (and A's) must be whole 16-byte chunks.
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 256, 256, 16, 256, 4, 4, "f32_mfma32_256x256x16_w2x2_a4b4_nt_ring4",
     &launch_f32_ring<4, 4, true>, 0, nullptr, kLayoutNT, false, kOutAll},
    // A stored K x M (and B either way): the stored rows of A^T (M long) are
    // 16-byte chunks too.
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 256, 256, 16, 256, 4, 4, "f32_mfma32_256x256x16_w2x2_a4b4_tn_ring4",
     &launch_f32_ring<4, 4, false, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 256, 256, 16, 256, 4, 4, "f32_mfma32_256x256x16_w2x2_a4b4_tt_ring4",
     &launch_f32_ring<4, 4, true, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    F32_TILED(256, 256, 16, 2, 2, 4, 4, 4),
    F32_TILED(256, 256, 16, 2, 2, 4, 1, 4),
    F32_TILED(256, 256, 16, 2, 2, 1, 4, 4),
    F32_TILED(256, 256, 16, 2, 2, 1, 1, 4),
    // 128 x 128 with B rows of whole 16-byte chunks: the ring, then the
    // register-staged kernels.
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 128, 128, 16, 256, 4, 4, "f32_mfma32_128x128x16_w2x2_a4b4_ring4",
     &launch_f32_ring64<4, 4, 2>, 0, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 128, 128, 16, 256, 1, 4, "f32_mfma32_128x128x16_w2x2_a1b4_ring4",
     &launch_f32_ring64<1, 4, 2>, 0, nullptr, kLayoutNN, false, kOutAll},
    F32_TILED(128, 128, 16, 2, 2, 4, 4, 8),
    F32_TILED(128, 128, 16, 2, 2, 4, 1, 8),
    F32_TILED(128, 128, 16, 2, 2, 1, 4, 8),
    F32_TILED(128, 128, 16, 2, 2, 1, 1, 8),
    // 128 x 128 and 64 x 64 rings with A or B stored transposed (the only
    // kernels of those tile sizes for those layouts).
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 128, 128, 16, 256, 4, 4, "f32_mfma32_128x128x16_w2x2_a4b4_nt_ring4",
     &launch_f32_ring64<4, 4, 2, true, false>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 128, 128, 16, 256, 4, 4, "f32_mfma32_128x128x16_w2x2_a4b4_tn_ring4",
     &launch_f32_ring64<4, 4, 2, false, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 128, 128, 16, 256, 4, 4, "f32_mfma32_128x128x16_w2x2_a4b4_tt_ring4",
     &launch_f32_ring64<4, 4, 2, true, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 64, 64, 16, 256, 4, 4, "f32_mfma32_64x64x16_w2x2_a4b4_nt_ring6",
     &launch_f32_ring64<4, 6, 1, true, false>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 64, 64, 16, 256, 4, 4, "f32_mfma32_64x64x16_w2x2_a4b4_tn_ring6",
     &launch_f32_ring64<4, 6, 1, false, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 64, 64, 16, 256, 4, 4, "f32_mfma32_64x64x16_w2x2_a4b4_tt_ring6",
     &launch_f32_ring64<4, 6, 1, true, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    // 64 x 64 with B rows of whole 16-byte chunks: the ring (A loaded 16 or 4
    // bytes per lane), then the register-staged kernels.
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 64, 64, 16, 256, 4, 4, "f32_mfma32_64x64x16_w2x2_a4b4_ring6",
     &launch_f32_ring64<4, 6, 1>, 0, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_TILED, 64, 64, 16, 256, 1, 4, "f32_mfma32_64x64x16_w2x2_a1b4_ring6",
     &launch_f32_ring64<1, 6, 1>, 0, nullptr, kLayoutNN, false, kOutAll},
    F32_TILED(64, 64, 16, 2, 2, 4, 4, 8),
    F32_TILED(64, 64, 16, 2, 2, 4, 1, 8),
    F32_TILED(64, 64, 16, 2, 2, 1, 4, 8),
    F32_TILED(64, 64, 16, 2, 2, 1, 1, 8),
};
const int kF32TiledKernelCount = sizeof(kF32TiledKernels) / sizeof(kF32TiledKernels[0]);
#endif

}  // namespace gemm
