// fp8 (OCP E4M3) GEMM, A untransposed (M x K) times B stored N x K, on the
// gfx950 matrix cores with A moved as whole 128-byte lines.
//
// This is the fp8 ring kernel of gemm_fp8_tiled.hip (a 64-byte k slice of
// each row feeds one v_mfma_f32_32x32x64_f8f6f4 per fragment pair) with A's
// panel loaded the way the whole-line bf16 kernel (gemm_bf16_lines.hip)
// loads it: 128 k at a time, a whole cache line per row, into one of three
// 32 KB "pair" stages that each serve two slices.  B keeps the ring's
// single-slice stages (four of 16 KB), 160 KB of LDS in all.  The line
// granularity is the coalescing rung of "A GEMM Kernel, Step by Step"
// taken to the cache line; the multi-stage asynchronous-copy ring is that
// page's "What is left", at the tensor-core level of "Tiled matrix
// multiplication" ("How it works").
//
//   A pair stage: [256 rows][8 chunks of 16 B] (128 k); logical chunk c of
//     row r sits at c ^ ((r >> 1) & 7).  A fragment read (32 consecutive
//     rows, one chunk each) then touches each 16-byte bank group of the
//     256-byte period exactly twice per half-wave.
//   B stage: [256 rows][4 chunks of 16 B] (64 k); chunk c of row r at
//     c ^ ((r >> 2) & 3), as in the ring.
//   Fragments: lane (h, l32) of a 32-row fragment holds bytes 32h .. 32h+31
//     of its row's slice, read as two 16-byte reads (logical chunks 2h and
//     2h+1 of the slice; 4*par + 2h and 4*par + 2h + 1 of A's pair row for
//     the slice of parity par).  The pairing of bytes and the order of the
//     sums are the ring's, so the two kernels give identical bits.
//
// Schedule, per slice kt (A pair stage (kt/2) % 3, B stage kt % 4, register
// set kt % 2): every wave waits for its own reads of slice kt and for slice
// kt+1 to land, then a barrier; then 16 matrix instructions on slice kt,
// each paired with one of the 16 fragment reads of slice kt+1 and, every
// other one, with one of the slice's 8 loads:
//   * B slice kt + 4 into stage kt % 4 (read during slice kt - 1, so free
//     after this slice's barrier), 4 loads;
//   * A pair (kt + 5) / 2, loads 0..3, when kt is odd, or pair (kt + 4) / 2,
//     loads 4..7, when kt is even, into stage pair % 3 (its previous pair's
//     last slice was read during slice 2*pair - 6, so it is free after the
//     barrier of slice 2*pair - 5).
// At the barrier of slice kt every load of slice kt - 3 or earlier has
// landed (vmcnt(16): slices kt - 2 and kt - 1 issued 8 each), which covers
// B slice kt + 1 and both halves of the A pair holding it.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm_lines.hpp"
#include "gemm.h"

namespace gemm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int fl_swz_a(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int fl_swz_b(int row) { return (row >> 2) & 3; }

template <int OUT>
__global__ void __launch_bounds__(256)
fp8_lines_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint8_t>(p);
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int kAPair = BM * 2 * BK;       // 32 KB: 256 rows x 128 k
    constexpr int kBSlice = BN * BK;          // 16 KB: 256 rows x 64 k
    constexpr int UNROLL = 12;                // stage cycles: A 3 pairs = 6 slices, B 4 slices, registers 2
    __shared__ __attribute__((aligned(1024))) char sa0[kAPair], sa1[kAPair], sa2[kAPair];
    __shared__ __attribute__((aligned(1024))) char sb0[kBSlice], sb1[kBSlice], sb2[kBSlice], sb3[kBSlice];
    auto a_stage = [&](int i) -> char * { return i == 0 ? sa0 : i == 1 ? sa1 : sa2; };
    auto b_stage = [&](int i) -> char * { return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : sb3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // A load j (0..7) of this wave for a pair: rows 8g .. 8g+7 with g =
    // 8*wave + j (lane -> row 8g + lane/8, physical chunk lane%8), landing at
    // stage + 1024 g.  B load j (0..3) of a slice: rows 16*(4*wave + j) ..
    // +15 (lane -> row 16*(4*wave + j) + lane/4, physical chunk lane%4),
    // landing at stage + 1024 (4*wave + j).
    uint32_t a_goff[8], b_goff[4];
    int a_kc[8], b_kc[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 8 * (8 * wave + j) + (lane >> 3);
        const int lc = (lane & 7) ^ fl_swz_a(row);
        a_kc[j] = 16 * lc;
        a_goff[j] = panel_off(row, a_rows, lda, 16 * lc, 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 16 * (4 * wave + j) + (lane >> 2);
        const int lc = (lane & 3) ^ fl_swz_b(row);
        b_kc[j] = 16 * lc;
        b_goff[j] = panel_off(row, b_rows, ldb, 16 * lc, 1);
    }
    // Resources of pair P of A (k 128P ..) and slice s of B (k 64s ..),
    // rebased per use: rows past M (N) read the last valid row, and a chunk
    // at or past K gets 2^31 added to its offset.
    auto rsrc_a = [&](int P) {
        const int k0 = 2 * BK * P;
        return make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent((int64_t)(a_rows - 1) * lda + (K - k0)));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent((int64_t)(b_rows - 1) * ldb + (K - k0)));
    };
    auto dma_a = [&](int P, int si, const rsrc_t &ra, int j) {
        const uint32_t poison = (uint32_t)(a_kc[j] >= K - 2 * BK * P) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(a_stage(si) + (8 * wave + j) * 1024), 16,
                                                 a_goff[j] + poison, 0, 0, 0);
    };
    auto dma_b = [&](int s, int si, const rsrc_t &rb, int j) {
        const uint32_t poison = (uint32_t)(b_kc[j] >= K - BK * s) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(b_stage(si) + (4 * wave + j) * 1024), 16,
                                                 b_goff[j] + poison, 0, 0, 0);
    };

    // Fragment reads.  Slot r (0..15) of a slice: r < 8 reads A fragment
    // r / 2, half r % 2; r >= 8 reads B fragment (r - 8) / 2, half r % 2.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int sa = fl_swz_a(l32), sb = fl_swz_b(l32);
    const uint32_t fa_row = (uint32_t)((wm * 128 + l32) * 2 * BK);
    const uint32_t fb_row = (uint32_t)((wn * 128 + l32) * BK);
    i32x8 fa[2][4], fb[2][4];
    auto read_slot = [&](int asi, int par, int bsi, int set, int r) {
        const int f = (r >> 1) & 3, hf = r & 1;
        u32x4 v;
        if (r < 8) {
            const int c = (4 * par + 2 * h + hf) ^ sa;
            v = *reinterpret_cast<const u32x4 *>(a_stage(asi) + fa_row + 32 * 2 * BK * f + 16 * c);
        } else {
            const int c = (2 * h + hf) ^ sb;
            v = *reinterpret_cast<const u32x4 *>(b_stage(bsi) + fb_row + 32 * BK * f + 16 * c);
        }
        i32x8 *frags = r < 8 ? fa[set] : fb[set];
#pragma unroll
        for (int e = 0; e < 4; ++e) frags[f][4 * hf + e] = (int)v[e];
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // B^T as the first operand and A^T as the second, as in the ring: each
    // lane then holds runs of 4 consecutive columns of one row of C.
    auto mma = [&](int set, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0, 0,
                                                                     0, 0);
    };

    // Prologue: A pairs 0 and 1, B slices 0..3, and A pair 2's loads 0..3
    // (the share of "slice -1"), in the order the waits below assume.
    const int nk = (K + BK - 1) / BK;
    {
        const rsrc_t ra0 = rsrc_a(0), ra1 = rsrc_a(1), ra2 = rsrc_a(2);
        const rsrc_t rb0 = rsrc_b(0), rb1 = rsrc_b(1), rb2 = rsrc_b(2), rb3 = rsrc_b(3);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma_a(0, 0, ra0, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(0, 0, rb0, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(1, 1, rb1, j);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma_a(1, 1, ra1, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(2, 2, rb2, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(3, 3, rb3, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(2, 2, ra2, j);
    }
    // Slice 0 (A pair 0, B slice 0) is followed by 24 loads.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(24));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) read_slot(0, 0, 0, 0, r);

    // Slice kt with u = kt % 12 a compile-time constant (the stages and the
    // register set follow from it).
    auto slice = [&](int u, int kt) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(16));
        __builtin_amdgcn_s_barrier();
        const int as_n = ((u + 1) >> 1) % 3, bs_n = (u + 1) % 4;     // stages of slice kt + 1
        const int PA = (u & 1) ? (kt + 5) >> 1 : (kt + 4) >> 1;    // the A pair this slice loads
        const int pa_st = ((u & 1) ? (u + 5) >> 1 : (u + 4) >> 1) % 3;
        const int ja = (u & 1) ? 0 : 4;                             // its loads ja .. ja+3
        const rsrc_t ra = rsrc_a(PA), rb = rsrc_b(kt + 4);          // zeros past the end
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            mma(u & 1, t);
            read_slot(as_n, (u + 1) & 1, bs_n, (u + 1) & 1, t);
            if ((t & 1) == 0) {
                const int q = t >> 1;
                if (q < 4) dma_b(kt + 4, u % 4, rb, q);
                else dma_a(PA, pa_st, ra, ja + q - 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Whole groups of 12 slices run as straight-line code, then the last
    // nk % 12 one by one (an exit test per slice would split the body into
    // blocks across which the compiler cannot tell which stage each load
    // writes, and it would wait for every load before each read).
    const int nfull = nk / UNROLL;
    int kb = 0;
    for (int it = 0; it < nfull; ++it, kb += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) slice(u, kb + u);
    }
    const int rem = nk - kb;
#pragma unroll
    for (int u = 0; u < UNROLL - 1; ++u)
        if (u < rem) slice(u, kb + u);
    // Every load (including those past K) has landed and every wave is done
    // with the stages before the epilogue reuses their memory.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    // Epilogue, in two passes of 64 columns per wave (lines_epilogue; N is
    // free): the wave's 32 KB of LDS is a pair stage for waves 0-2 and two B
    // stages for wave 3.
    char *stg = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : nullptr;
    lines_epilogue<OUT, true>(p, acc, [&](int row) -> char * {
        return stg != nullptr ? stg + row * 256 : (row < 64 ? sb0 : sb1) + (row & 63) * 256;
    }, m0, n0, wm, wn, lane);
}

// The same ring at a quarter of the tile: 128 x 128 outputs per workgroup,
// each wave 64 x 64 (2 x 2 fragments), for problems with too few 256 x 256
// tiles to fill the compute units.  Three A pair stages of 16 KB (128 rows x
// 128 k) and four B stages of 8 KB (128 rows x 64 k), 80 KB in all, so that
// two workgroups fit a compute unit.  Per slice, 4 matrix instructions per
// wave, each paired with two of the 8 fragment reads of the next slice and
// one of the slice's 4 loads: B slice kt + 4 (loads 0, 1), then A pair
// (kt + 5) / 2 loads 0, 1 when kt is odd or pair (kt + 4) / 2 loads 2, 3 when
// kt is even.  At the barrier of slice kt every load of slice kt - 3 or
// earlier has landed (vmcnt(8)), which covers slice kt + 1.  Layouts,
// swizzles and the per-lane order of the sums are the 256 x 256 kernel's, so
// the two give identical bits.
template <int OUT>
__global__ void __launch_bounds__(256)
fp8_lines128_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint8_t>(p);
    constexpr int BM = 128, BN = 128, BK = 64;
    constexpr int kAPair = BM * 2 * BK;       // 16 KB: 128 rows x 128 k
    constexpr int kBSlice = BN * BK;          // 8 KB: 128 rows x 64 k
    constexpr int UNROLL = 12;
    __shared__ __attribute__((aligned(1024))) char sa0[kAPair], sa1[kAPair], sa2[kAPair];
    __shared__ __attribute__((aligned(1024))) char sb0[kBSlice], sb1[kBSlice], sb2[kBSlice], sb3[kBSlice];
    auto a_stage = [&](int i) -> char * { return i == 0 ? sa0 : i == 1 ? sa1 : sa2; };
    auto b_stage = [&](int i) -> char * { return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : sb3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // A load j (0..3) for a pair: rows 8g .. 8g+7 with g = 4*wave + j (lane ->
    // row 8g + lane/8, physical chunk lane%8), landing at stage + 1024 g.  B
    // load j (0..1) of a slice: rows 16g .. 16g+15 with g = 2*wave + j (lane
    // -> row 16g + lane/4, physical chunk lane%4), landing at stage + 1024 g.
    uint32_t a_goff[4], b_goff[2];
    int a_kc[4], b_kc[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 8 * (4 * wave + j) + (lane >> 3);
        const int lc = (lane & 7) ^ fl_swz_a(row);
        a_kc[j] = 16 * lc;
        a_goff[j] = panel_off(row, a_rows, lda, 16 * lc, 1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * (2 * wave + j) + (lane >> 2);
        const int lc = (lane & 3) ^ fl_swz_b(row);
        b_kc[j] = 16 * lc;
        b_goff[j] = panel_off(row, b_rows, ldb, 16 * lc, 1);
    }
    auto rsrc_a = [&](int P) {
        const int k0 = 2 * BK * P;
        return make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent((int64_t)(a_rows - 1) * lda + (K - k0)));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent((int64_t)(b_rows - 1) * ldb + (K - k0)));
    };
    auto dma_a = [&](int P, int si, const rsrc_t &ra, int j) {
        const uint32_t poison = (uint32_t)(a_kc[j] >= K - 2 * BK * P) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(a_stage(si) + (4 * wave + j) * 1024), 16,
                                                 a_goff[j] + poison, 0, 0, 0);
    };
    auto dma_b = [&](int s, int si, const rsrc_t &rb, int j) {
        const uint32_t poison = (uint32_t)(b_kc[j] >= K - BK * s) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(b_stage(si) + (2 * wave + j) * 1024), 16,
                                                 b_goff[j] + poison, 0, 0, 0);
    };

    // Fragment reads.  Slot r (0..7) of a slice: r < 4 reads A fragment r / 2,
    // half r % 2; r >= 4 reads B fragment (r - 4) / 2, half r % 2.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int sa = fl_swz_a(l32), sb = fl_swz_b(l32);
    const uint32_t fa_row = (uint32_t)((wm * 64 + l32) * 2 * BK);
    const uint32_t fb_row = (uint32_t)((wn * 64 + l32) * BK);
    i32x8 fa[2][2], fb[2][2];
    auto read_slot = [&](int asi, int par, int bsi, int set, int r) {
        const int f = (r >> 1) & 1, hf = r & 1;
        u32x4 v;
        if (r < 4) {
            const int c = (4 * par + 2 * h + hf) ^ sa;
            v = *reinterpret_cast<const u32x4 *>(a_stage(asi) + fa_row + 32 * 2 * BK * f + 16 * c);
        } else {
            const int c = (2 * h + hf) ^ sb;
            v = *reinterpret_cast<const u32x4 *>(b_stage(bsi) + fb_row + 32 * BK * f + 16 * c);
        }
        i32x8 *frags = r < 4 ? fa[set] : fb[set];
#pragma unroll
        for (int e = 0; e < 4; ++e) frags[f][4 * hf + e] = (int)v[e];
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

    // Prologue: A pairs 0 and 1, B slices 0..3, and A pair 2's loads 0, 1 (the
    // share of "slice -1"); slice 0 (A pair 0, B slice 0) is followed by 12.
    const int nk = (K + BK - 1) / BK;
    {
        const rsrc_t ra0 = rsrc_a(0), ra1 = rsrc_a(1), ra2 = rsrc_a(2);
        const rsrc_t rb0 = rsrc_b(0), rb1 = rsrc_b(1), rb2 = rsrc_b(2), rb3 = rsrc_b(3);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(0, 0, ra0, j);
        dma_b(0, 0, rb0, 0);
        dma_b(0, 0, rb0, 1);
        dma_b(1, 1, rb1, 0);
        dma_b(1, 1, rb1, 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(1, 1, ra1, j);
        dma_b(2, 2, rb2, 0);
        dma_b(2, 2, rb2, 1);
        dma_b(3, 3, rb3, 0);
        dma_b(3, 3, rb3, 1);
        dma_a(2, 2, ra2, 0);
        dma_a(2, 2, ra2, 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(12));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 8; ++r) read_slot(0, 0, 0, 0, r);

    auto slice = [&](int u, int kt) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));
        __builtin_amdgcn_s_barrier();
        const int as_n = ((u + 1) >> 1) % 3, bs_n = (u + 1) % 4;
        const int PA = (u & 1) ? (kt + 5) >> 1 : (kt + 4) >> 1;
        const int pa_st = ((u & 1) ? (u + 5) >> 1 : (u + 4) >> 1) % 3;
        const int ja = (u & 1) ? 0 : 2;
        const rsrc_t ra = rsrc_a(PA), rb = rsrc_b(kt + 4);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            mma(u & 1, t);
            read_slot(as_n, (u + 1) & 1, bs_n, (u + 1) & 1, 2 * t);
            read_slot(as_n, (u + 1) & 1, bs_n, (u + 1) & 1, 2 * t + 1);
            if (t < 2) dma_b(kt + 4, u % 4, rb, t);
            else dma_a(PA, pa_st, ra, ja + t - 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nfull = nk / UNROLL;
    int kb = 0;
    for (int it = 0; it < nfull; ++it, kb += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) slice(u, kb + u);
    }
    const int rem = nk - kb;
#pragma unroll
    for (int u = 0; u < UNROLL - 1; ++u)
        if (u < rem) slice(u, kb + u);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    // Epilogue in one pass of 64 columns per wave: 16 KB of staging each, a
    // pair stage for waves 0-2 and two B stages for wave 3.
    char *stg = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : nullptr;
    lines_epilogue<OUT, true>(p, acc, [&](int row) -> char * {
        return stg != nullptr ? stg + row * 256 : (row < 32 ? sb0 : sb1) + (row & 31) * 256;
    }, m0, n0, wm, wn, lane);
}

hipError_t launch_fp8_lines(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&fp8_lines_kernel<GEMM_OUT_BF16>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&fp8_lines_kernel<GEMM_OUT_FP8>)
                                           : reinterpret_cast<const void *>(&fp8_lines_kernel<GEMM_OUT_F32>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

hipError_t launch_fp8_lines128(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 127) / 128, tiles_n = (p.N + 127) / 128;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&fp8_lines128_kernel<GEMM_OUT_BF16>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&fp8_lines128_kernel<GEMM_OUT_FP8>)
                                           : reinterpret_cast<const void *>(&fp8_lines128_kernel<GEMM_OUT_F32>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

template __global__ void fp8_lines_kernel<GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void fp8_lines128_kernel<GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void fp8_lines128_kernel<GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void fp8_lines128_kernel<GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void fp8_lines_kernel<GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void fp8_lines_kernel<GEMM_OUT_FP8>(GemmParams, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// tile_k is the depth of one A load (a pair of 64-deep slices); K from 1024.
const KernelDesc kFp8LinesKernels[] = {
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 256, 256, 128, 256, 16, 16, "fp8_mfma32_256x256x128_w2x2_nt_lines",
     &launch_fp8_lines, 1024, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_TILED, 128, 128, 128, 256, 16, 16, "fp8_mfma32_128x128x128_w2x2_nt_lines",
     &launch_fp8_lines128, 256, nullptr, kLayoutNT, false, kOutAll},
};
const int kFp8LinesKernelCount = sizeof(kFp8LinesKernels) / sizeof(kFp8LinesKernels[0]);
#endif

}  // namespace gemm
