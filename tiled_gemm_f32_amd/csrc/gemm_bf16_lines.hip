// bf16-operand, fp32-accumulate GEMM on the gfx950 matrix cores: the
// 256 x 256 ring kernel of gemm_bf16_tiled.hip with every global access made
// of whole 128-byte lines.
//
// The ring kernel loads 32 k of each row of A per slice (64 bytes, half a
// cache line) and B in 32-column blocks (again 64 bytes per row), and its
// epilogue stores 32 bytes per row per instruction.  Every one of those
// partial-line requests occupies the memory pipeline like a whole line, and
// with A and B missing in L2 most of the time (each panel is read by a few
// compute units and then evicted) the loads, not the matrix cores, set the
// pace.  Here:
//   * A is loaded 64 k at a time, a full 128-byte line per row, into one of
//     three 32 KB "pair" stages (256 rows x 64 k); each pair serves two 32-deep
//     compute slices.
//   * B is loaded per 32-deep slice into one of four 16 KB stages as four
//     64-column blocks, each row of a block a full 128-byte line.
//   * The epilogue passes each wave's accumulators through LDS so that every
//     store instruction writes four rows of 256 contiguous bytes.
// The compute schedule is the ring kernel's: each 32-deep slice is two blocks
// of 16 matrix instructions per wave (a 128 x 128 accumulator tile), with the
// fragment reads of the next half-slice and the refill loads pinned between
// them, and one barrier per slice.  The refill loads are spread evenly: every
// block issues two of A and two of B.  This is the blocked method of "Tiled
// matrix multiplication" ("How it works", down to its tensor-core level) with
// the multi-stage asynchronous-copy pipeline of "A GEMM Kernel, Step by Step"
// ("What is left"); the line-granular transfers are its coalescing rung taken
// to the cache line.
//
// LDS layouts (16-byte chunks XOR-swizzled so that the reads below touch
// every bank group equally):
//   A pair stage: [256 rows][8 chunks]; logical chunk c (k = 8c .. 8c+7 of
//     the pair) of row r sits at chunk c ^ ((r >> 1) & 7).  A fragment read
//     (32 consecutive rows, one chunk each) then hits each 16-byte bank group
//     of the 256-byte period exactly twice per half-wave.
//   B stage: [4 blocks of 64 columns][32 k rows][8 chunks]; chunk c of k row
//     r sits at c ^ (4 * ((r >> 1) & 1)).  The transposing reads
//     (ds_read_b64_tr_b16: 4 k rows x 16 columns per 16 lanes) then touch 16
//     distinct bank groups per half-wave.
//   Epilogue staging, per wave: [128 rows][16 chunks of 4 floats]; chunk c of
//     row r sits at c ^ (r & 15), for both the accumulator-layout writes and
//     the row-major reads.
// Each lane accumulates every output it owns over k in the same order as the
// ring kernel, so the two give identical bits.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm_lines.hpp"
#include "gemm.h"

namespace gemm {
namespace {

__device__ __forceinline__ int lines_swz_a(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lines_swz_b(int row) { return 4 * ((row >> 1) & 1); }

template <int OUT, bool BT>
__global__ void __launch_bounds__(256)
bf16_lines_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 256, BN = 256, BK = 32;
    constexpr int kAPair = BM * 2 * BK * 2;   // 32 KB: 256 rows x 64 k
    constexpr int kBSlice = BK * BN * 2;      // 16 KB: 32 k rows x 256 columns
    constexpr int UNROLL = 12;                // stage cycles: A 3 pairs = 6 slices, B 4 slices
    // One array per stage: the compiler can then tell that a fragment read of
    // one stage does not depend on loads still landing in another.
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
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // A load j (0..7) of this wave for a pair: rows 8g .. 8g+7 with g = 8*wave
    // + j (lane -> row 8g + lane/8, physical chunk lane%8), landing at
    // stage + 1024 g.  B load j (0..3) of a slice: block `wave` (columns
    // 64*wave ..), k rows 8j .. 8j+7 (lane -> row 8j + lane/8), landing at
    // stage + 4096 wave + 1024 j.
    uint32_t a_goff[8], b_goff[4];
    int a_kc[8], b_kc[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 8 * (8 * wave + j) + (lane >> 3);
        const int lc = (lane & 7) ^ lines_swz_a(row);
        a_kc[j] = 8 * lc;
        a_goff[j] = panel_off(row, a_rows, lda, 8 * lc, 2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (BT) {
            // B stored N x K: its slice is 256 rows (columns of C) of 64
            // bytes, laid out as the ring kernel lays out A's slice (chunk
            // c of row r at c ^ ((r >> 2) & 3)); load j fills rows
            // 16*(4*wave + j) .. +15 (lane -> row 16*(4*wave + j) + lane/4).
            const int row = 16 * (4 * wave + j) + (lane >> 2);
            const int lc = (lane & 3) ^ ((row >> 2) & 3);
            b_kc[j] = 8 * lc;
            b_goff[j] = panel_off(row, b_rows, ldb, 8 * lc, 2);
        } else {
            const int row = 8 * j + (lane >> 3);
            const int lc = (lane & 7) ^ lines_swz_b(row);
            b_kc[j] = 0;
            b_goff[j] = (uint32_t)(row * ldb + 64 * wave + 8 * lc) * 2u;
        }
    }
    // Resources: pair P of A (k 64P ..) and slice s of B (k rows 32s ..),
    // rebased per use.  k rows past K fall outside B's extent; A chunks at or
    // past K get 2^31 added to their offset; rows past M read row M - 1.
    auto rsrc_a = [&](int P) {
        const int k0 = 2 * BK * P;
        return make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 2));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        if (BT)
            return make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent(((int64_t)(b_rows - 1) * ldb + (K - k0)) * 2));
        return make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
    };
    auto dma_a = [&](int P, int si, const rsrc_t &ra, int j) {
        char *stage = a_stage(si);
        const uint32_t poison = (uint32_t)(a_kc[j] >= K - 2 * BK * P) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(stage + (8 * wave + j) * 1024), 16,
                                                 a_goff[j] + poison, 0, 0, 0);
    };
    auto dma_b = [&](int s, int si, const rsrc_t &rb, int j) {
        char *stage = b_stage(si);
        if (BT) {
            // A chunk at or past K in a valid row would read the next row.
            const uint32_t poison = (uint32_t)(b_kc[j] >= K - BK * s) << 31;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(stage + 1024 * (4 * wave + j)), 16,
                                                     b_goff[j] + poison, 0, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(stage + 4096 * wave + 1024 * j), 16, b_goff[j],
                                                     0, 0, 0);
        }
    };

    // Fragment reads.  A fragment f, k half s of a slice with pair parity
    // par: row wm*128 + 32f + l32, logical chunk 4*par + 2s + h.  B fragment
    // f (columns wn*128 + 32f .. +31: block 2*wn + f/2, bytes 64*(f%2) ..),
    // k half s: lane (q, j16) points at k row 16s + 8*(q/2) + j16/4 (and 4
    // rows on for the second read), columns 16*(q%2) + 4*(j16%4) .. +3.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int a_sw = lines_swz_a(l32);
    const uint32_t fa_row = (uint32_t)((wm * 128 + l32) * 128);
    const int q = lane >> 4, j16 = lane & 15;
    const int brow = 8 * (q >> 1) + (j16 >> 2);
    const int bx = 2 * (q & 1) + ((j16 & 3) >> 1);          // logical chunk, bits 0-1
    const int bsw = (j16 >> 3) & 1;                          // = ((brow >> 1) & 1)
    uint32_t fb_off[2];                                      // by fragment parity f % 2
#pragma unroll
    for (int fp = 0; fp < 2; ++fp)
        fb_off[fp] = (uint32_t)(wn * 2 * 4096 + brow * 128 + 16 * (bx + 4 * (fp ^ bsw)) + 8 * (j16 & 1));
    // B stored N x K: fragment f, k half s is row wn*128 + 32f + l32 of the
    // slice, logical chunk 2s + h (16-byte reads, as the ring kernel reads A).
    uint32_t fbt_off[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
        fbt_off[s2] = (uint32_t)((wn * 128 + l32) * 64 + 16 * ((2 * s2 + h) ^ ((l32 >> 2) & 3)));

    bf16x8 fa[2][4], fb[2][4];
    // Read slot r (0..7) of half s of slice (A stage asi, parity par; B stage
    // bsi) into register set `set`, in the order the next block of matrix
    // instructions consumes them: A0, B0, B1, B2, B3, A1, A2, A3.
    auto read_slot = [&](int asi, int par, int bsi, int s, int set, int r) {
        char *as = a_stage(asi), *bs = b_stage(bsi);
        if (r == 0 || r >= 5) {
            const int f = r == 0 ? 0 : r - 4;
            const int c = (4 * par + 2 * s + h) ^ a_sw;
            fa[set][f] = *reinterpret_cast<const bf16x8 *>(as + fa_row + 4096 * f + 16 * c);
        } else if (BT) {
            const int f = r - 1;
            fb[set][f] = *reinterpret_cast<const bf16x8 *>(bs + fbt_off[s] + 2048 * f);
        } else {
            const int f = r - 1;
            const uint32_t off = fb_off[f & 1] + 4096 * (f >> 1) + 2048 * s;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(bs + off));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(bs + off + 512));
            fb[set][f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // B^T as the first operand and A^T as the second (C^T = B^T A^T): each
    // lane holds runs of 4 consecutive columns of one row of C.
    auto mma = [&](int set, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Load plan (per wave; every block of 16 matrix instructions issues two A
    // and two B loads):
    //   B slice s: loads 0, 1 in block 2 of slice s - 4, loads 2, 3 in block 1
    //     of slice s - 3, into stage s % 4 (free since the barrier of slice
    //     s - 4, after which it is no longer read).
    //   A pair P: quarter q (loads 2q, 2q + 1) in block 2 of slice 2P - 5,
    //     blocks 1 and 2 of slice 2P - 4 and block 1 of slice 2P - 3, into
    //     stage P % 3 (free since the barrier of slice 2P - 5).
    // At the barrier of slice kt every wave needs slice kt + 1's B and the A
    // pair holding it.  The last of those loads is issued in block 1 of slice
    // kt - 2 or earlier, and 16 loads per lane follow it by then: vmcnt(16).
    // The prologue issues the loads of "slices" -5 .. -1 in the same order.
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
        dma_a(2, 2, ra2, 0);
        dma_a(2, 2, ra2, 1);
        dma_b(3, 3, rb3, 0);
        dma_b(3, 3, rb3, 1);
    }
    // Resources carried into the next block: B slice kt + 3 and A pair
    // (kt + 4) / 2, for block 1 of slice kt.
    rsrc_t rb_pend = rsrc_b(3), ra_pend = rsrc_a(2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(20));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 8; ++r) read_slot(0, 0, 0, 0, 0, r);
    // Slice kt, with u = kt % 12 a compile-time constant in every call below
    // (the stage of each operand follows from it).
    auto slice = [&](int u, int kt) {
        const int as = (u >> 1) % 3, bs = u % 4;
        // Block 1: the slice's second k half; reads of that half; loads of A
        // pair (kt + 4) / 2 (quarter 3 or 1) and B slice kt + 3 (loads 2, 3);
        // resources of the block-2 loads.
        const int a1 = ((u + 4) >> 1) % 3, b1 = (u + 3) % 4;
        const int q1 = (u & 1) ? 3 : 1;
        const int P1 = (kt + 4) >> 1, P2 = (kt + 5) >> 1;
        rsrc_t ra_next, rb_next;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            mma(0, t);
            if (t < 8) read_slot(as, u & 1, bs, 1, 1, t);
            else if (t == 9) dma_a(P1, a1, ra_pend, 2 * q1);
            else if (t == 11) dma_b(kt + 3, b1, rb_pend, 2);
            else if (t == 13) dma_a(P1, a1, ra_pend, 2 * q1 + 1);
            else if (t == 15) dma_b(kt + 3, b1, rb_pend, 3);
            else if (t == 8) ra_next = rsrc_a(P2);
            else if (t == 10) rb_next = rsrc_b(kt + 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(16));
        __builtin_amdgcn_s_barrier();
        // Block 2: the slice's second k half is multiplied while the first k
        // half of slice kt + 1 is read; loads of A pair (kt + 5) / 2 (quarter
        // 0 or 2) and B slice kt + 4 (loads 0, 1).
        const int a2 = ((u + 5) >> 1) % 3, b2 = u % 4;
        const int as_n = ((u + 1) >> 1) % 3, bs_n = (u + 1) % 4;
        const int q2 = (u & 1) ? 0 : 2;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            mma(1, t);
            if (t & 1) read_slot(as_n, (u + 1) & 1, bs_n, 0, 0, t >> 1);
            else if (t == 0) dma_a(P2, a2, ra_next, 2 * q2);
            else if (t == 2) dma_b(kt + 4, b2, rb_next, 0);
            else if (t == 4) dma_a(P2, a2, ra_next, 2 * q2 + 1);
            else if (t == 6) dma_b(kt + 4, b2, rb_next, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        rb_pend = rb_next;
        ra_pend = ra_next;
    };
    // Whole groups of 12 slices run as straight-line code (an exit test per
    // slice splits the body into blocks across which the compiler can no
    // longer tell which stage each load writes, and it then waits for every
    // load before each read); the last nk % 12 slices follow one by one.
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
    // with the ring before the epilogue reuses its memory.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    // Epilogue, in two passes of 64 columns per wave (lines_epilogue): the
    // wave's 32 KB of LDS is a pair stage for waves 0-2 and two B stages for
    // wave 3.
    char *stg = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : nullptr;
    lines_epilogue<OUT, BT>(p, acc, [&](int row) -> char * {
        return stg != nullptr ? stg + row * 256 : (row < 64 ? sb0 : sb1) + (row & 63) * 256;
    }, m0, n0, wm, wn, lane);
}

// The same ring at a quarter of the tile: 128 x 128 outputs per workgroup,
// each wave 64 x 64 (2 x 2 fragments), for problems with too few 256 x 256
// tiles to fill the compute units.  NA = 3 A-pair stages of 16 KB (128 rows
// x 64 k) and NB = 4 B-slice stages of 8 KB (two 64-column blocks of 32 k
// rows), 80 KB in all, so that two workgroups fit a compute unit.  Every
// block of 4 matrix instructions per wave issues one A and one B load; the
// LDS layouts, the swizzles and the per-lane order of accumulation are those
// of the 256 x 256 kernel.  BT: B stored N x K (its slices take that
// kernel's B-transposed layout and reads, and N is free); otherwise K x N.
//
// Deeper rings (4 + 6, 4 + 8 and 5 + 10 stages, up to the whole 160 KB of
// LDS, one workgroup per compute unit) were no faster even on a single wave
// of tiles (2048^3: 26.2 us here, 27.4-28.6 us deeper), so load latency is
// not what holds this kernel back; its 64 x 64 wave tile reads twice the LDS
// bytes per matrix instruction of the 256 x 256 kernel's 128 x 128 one.
template <int OUT, bool BT>
__global__ void __launch_bounds__(256)
bf16_lines128_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 128, BN = 128, BK = 32;
    constexpr int NA = 3, NB = 4;
    constexpr int kAPair = BM * 2 * BK * 2;   // 16 KB: 128 rows x 64 k
    constexpr int kBSlice = BK * BN * 2;      // 8 KB: 32 k rows x 128 columns
    constexpr int UNROLL = 12;                // 2 * NA slices per A cycle, NB per B cycle
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
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // A load j (0..3) of this wave for a pair: rows 8g .. 8g+7 with g = 4*wave
    // + j (lane -> row 8g + lane/8, physical chunk lane%8), landing at stage +
    // 1024 g.  B load j (0..1) of a slice: g = 2*wave + j covers block g/4
    // (columns 64*(g/4) ..), k rows 8*(g%4) .. +7 (lane -> k row 8*(g%4) +
    // lane/8), landing at stage + 1024 g.  B stored N x K: a slice is 128 rows
    // (columns of C) of 64 bytes, chunk c of row r at c ^ ((r >> 2) & 3), and
    // load j fills rows 16g .. 16g+15 (lane -> row 16g + lane/4).
    uint32_t a_goff[4], b_goff[2];
    int a_kc[4], b_kc[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 8 * (4 * wave + j) + (lane >> 3);
        const int lc = (lane & 7) ^ lines_swz_a(row);
        a_kc[j] = 8 * lc;
        a_goff[j] = panel_off(row, a_rows, lda, 8 * lc, 2);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int g = 2 * wave + j;
        if (BT) {
            const int row = 16 * g + (lane >> 2);
            const int lc = (lane & 3) ^ ((row >> 2) & 3);
            b_kc[j] = 8 * lc;
            b_goff[j] = panel_off(row, b_rows, ldb, 8 * lc, 2);
        } else {
            const int row = 8 * (g & 3) + (lane >> 3);
            const int lc = (lane & 7) ^ lines_swz_b(row);
            b_kc[j] = 0;
            b_goff[j] = (uint32_t)(row * ldb + 64 * (g >> 2) + 8 * lc) * 2u;
        }
    }
    // Resources: pair P of A (k 64P ..) and slice s of B (k rows 32s ..),
    // rebased per use.  k rows past K fall outside B's extent; A chunks at or
    // past K get 2^31 added to their offset; rows past M read row M - 1.
    auto rsrc_a = [&](int P) {
        const int k0 = 2 * BK * P;
        return make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 2));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        if (BT)
            return make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent(((int64_t)(b_rows - 1) * ldb + (K - k0)) * 2));
        return make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
    };
    auto dma_a = [&](int P, int si, const rsrc_t &ra, int j) {
        const uint32_t poison = (uint32_t)(a_kc[j] >= K - 2 * BK * P) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(a_stage(si) + (4 * wave + j) * 1024), 16,
                                                 a_goff[j] + poison, 0, 0, 0);
    };
    auto dma_b = [&](int s, int si, const rsrc_t &rb, int j) {
        // B stored N x K: a chunk at or past K in a valid row would read the
        // next row.
        const uint32_t poison = BT ? (uint32_t)(b_kc[j] >= K - BK * s) << 31 : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(b_stage(si) + 1024 * (2 * wave + j)), 16,
                                                 b_goff[j] + poison, 0, 0, 0);
    };

    // Fragment reads, as in the 256 x 256 kernel: A fragment f, k half s of a
    // slice with pair parity par is row wm*64 + 32f + l32, logical chunk 4*par
    // + 2s + h; B fragment f (columns wn*64 + 32f ..: block wn, bytes 64f ..)
    // is read with two transposing reads per k half.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int a_sw = lines_swz_a(l32);
    const uint32_t fa_row = (uint32_t)((wm * 64 + l32) * 128);
    const int q = lane >> 4, j16 = lane & 15;
    const int brow = 8 * (q >> 1) + (j16 >> 2);
    const int bx = 2 * (q & 1) + ((j16 & 3) >> 1);
    const int bsw = (j16 >> 3) & 1;
    uint32_t fb_off[2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
        fb_off[f] = (uint32_t)(wn * 4096 + brow * 128 + 16 * (bx + 4 * (f ^ bsw)) + 8 * (j16 & 1));
    // B stored N x K: fragment f, k half s is row wn*64 + 32f + l32 of the
    // slice, logical chunk 2s + h.
    uint32_t fbt_off[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
        fbt_off[s2] = (uint32_t)((wn * 64 + l32) * 64 + 16 * ((2 * s2 + h) ^ ((l32 >> 2) & 3)));

    bf16x8 fa[2][2], fb[2][2];
    // Read slot r (0..3) in the order the next block consumes them: A0, B0,
    // B1, A1.
    auto read_slot = [&](int asi, int par, int bsi, int s, int set, int r) {
        if (r == 0 || r == 3) {
            const int f = r == 0 ? 0 : 1;
            const int c = (4 * par + 2 * s + h) ^ a_sw;
            fa[set][f] = *reinterpret_cast<const bf16x8 *>(a_stage(asi) + fa_row + 4096 * f + 16 * c);
        } else if (BT) {
            fb[set][r - 1] = *reinterpret_cast<const bf16x8 *>(b_stage(bsi) + fbt_off[s] + 2048 * (r - 1));
        } else {
            const int f = r - 1;
            const char *bp = b_stage(bsi) + fb_off[f] + 2048 * s;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)bp);
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(bp + 512));
            fb[set][f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto mma = [&](int set, int t) {
        const int i = t >> 1, j = t & 1;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Load plan (per wave), the 256 x 256 kernel's with one load where that
    // kernel issues two:
    //   B slice s (loads 0, 1) into stage s % NB: load 0 in block 2 of slice
    //     s - NB, load 1 in block 1 of slice s - NB + 1 (the stage is free
    //     from the barrier of slice s - NB, the last that reads it).
    //   A pair P (loads 0..3) into stage P % NA: load 0 in block 2 of slice
    //     2P - 2NA + 1, loads 1 and 2 in blocks 1 and 2 of the next slice,
    //     load 3 in block 1 of the one after (free from the barrier of slice
    //     2P - 2NA + 1, the last that reads pair P - NA).
    // The last load that slice kt + 1 needs is issued in block 1 of slice kt -
    // 2 or earlier, and 8 loads per lane follow it by the barrier of slice kt.
    // The prologue issues, in order, pair i then B slices 2i and 2i + 1 for i
    // = 0 .. NA - 1, each as far as the plan has it issued before slice 0;
    // slice 0 needs pair 0 and B slice 0, the first six loads.
    constexpr int kWait = 8;
    constexpr int kPrologue = 4 * (NA - 1) + 1 + 2 * (NB - 1) + 1;
    const int nk = (K + BK - 1) / BK;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const rsrc_t ra = rsrc_a(i);
#pragma unroll
        for (int j = 0; j < (i < NA - 1 ? 4 : 1); ++j) dma_a(i, i, ra, j);
#pragma unroll
        for (int s2 = 2 * i; s2 < 2 * i + 2; ++s2) {
            if (s2 >= NB) continue;
            const rsrc_t rb = rsrc_b(s2);
            dma_b(s2, s2, rb, 0);
            if (s2 < NB - 1) dma_b(s2, s2, rb, 1);
        }
    }
    rsrc_t rb_pend = rsrc_b(NB - 1), ra_pend = rsrc_a(NA - 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kPrologue - 6));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 4; ++r) read_slot(0, 0, 0, 0, 0, r);
    // Slice kt, with u = kt % UNROLL a compile-time constant in every call.
    auto slice = [&](int u, int kt) {
        const int as = (u >> 1) % NA, bs = u % NB;
        const int a1 = ((u + 2 * NA - 2) >> 1) % NA, b1 = (u + NB - 1) % NB;
        const int q1 = (u & 1) ? 3 : 1;
        const int P1 = (kt + 2 * NA - 2) >> 1, P2 = (kt + 2 * NA - 1) >> 1;
        rsrc_t ra_next, rb_next;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            mma(0, t);
            read_slot(as, u & 1, bs, 1, 1, t);
            if (t == 0) ra_next = rsrc_a(P2);
            else if (t == 1) dma_a(P1, a1, ra_pend, q1);
            else if (t == 2) rb_next = rsrc_b(kt + NB);
            else dma_b(kt + NB - 1, b1, rb_pend, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kWait));
        __builtin_amdgcn_s_barrier();
        const int a2 = ((u + 2 * NA - 1) >> 1) % NA, b2 = u % NB;
        const int as_n = ((u + 1) >> 1) % NA, bs_n = (u + 1) % NB;
        const int q2 = (u & 1) ? 0 : 2;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            mma(1, t);
            read_slot(as_n, (u + 1) & 1, bs_n, 0, 0, t);
            if (t == 0) dma_a(P2, a2, ra_next, q2);
            else if (t == 2) dma_b(kt + NB, b2, rb_next, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        rb_pend = rb_next;
        ra_pend = ra_next;
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
    // pair stage for waves 0-2 and two B slices for wave 3.
    char *stg = wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : nullptr;
    lines_epilogue<OUT, BT>(p, acc, [&](int row) -> char * {
        return stg != nullptr ? stg + row * 256 : (row < 32 ? sb0 : sb1) + (row & 31) * 256;
    }, m0, n0, wm, wn, lane);
}

// A stored K x M (m contiguous; the weight-gradient product X^T dY) times an
// untransposed B.  A's 32-deep slice then has the shape of B's (32 k rows of
// 256 columns), so both operands take the B machinery of the kernel above:
// four 16 KB single-slice stages each, loaded as four 64-column blocks whose
// rows are whole 128-byte lines, and read with the transposing
// ds_read_b64_tr_b16 (which gives each lane its k values in the order the
// 16-byte reads of an untransposed A do, so the bits equal the A^T ring's).
// Every block of 16 matrix instructions issues two loads of A and two of B,
// as above, with B's timing for both: slice s's loads 0, 1 in block 2 of
// slice s - 4 and loads 2, 3 in block 1 of slice s - 3, so the wait of
// vmcnt(16) at each barrier is unchanged.  128 KB of LDS.
template <int OUT>
__global__ void __launch_bounds__(256)
bf16_lines_tn_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 256, BN = 256, BK = 32;
    constexpr int kSlice = BK * 256 * 2;      // 16 KB: 32 k rows x 256 columns
    constexpr int UNROLL = 4;                 // stage cycle (and twice the register-set cycle)
    __shared__ __attribute__((aligned(1024))) char sa0[kSlice], sa1[kSlice], sa2[kSlice], sa3[kSlice];
    __shared__ __attribute__((aligned(1024))) char sb0[kSlice], sb1[kSlice], sb2[kSlice], sb3[kSlice];
    auto a_stage = [&](int i) -> char * { return i == 0 ? sa0 : i == 1 ? sa1 : i == 2 ? sa2 : sa3; };
    auto b_stage = [&](int i) -> char * { return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : sb3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    // Load j (0..3) of a slice, for either operand: block `wave` (columns
    // 64*wave ..), k rows 8j .. 8j+7 (lane -> row 8j + lane/8, physical chunk
    // lane%8), landing at stage + 4096 wave + 1024 j.  Columns past M (N)
    // belong to rows (columns) of C that are never stored.
    uint32_t a_goff[4], b_goff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int lc = (lane & 7) ^ lines_swz_b(row);
        a_goff[j] = (uint32_t)(row * lda + 64 * wave + 8 * lc) * 2u;
        b_goff[j] = (uint32_t)(row * ldb + 64 * wave + 8 * lc) * 2u;
    }
    // Resources of slice s, rebased per slice; k rows past K fall outside.
    auto rsrc_a = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent(((int64_t)(K - k0 - 1) * lda + (M - m0)) * 2));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
    };
    auto dma_a = [&](int si, const rsrc_t &ra, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(a_stage(si) + 4096 * wave + 1024 * j), 16,
                                                 a_goff[j], 0, 0, 0);
    };
    auto dma_b = [&](int si, const rsrc_t &rb, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(b_stage(si) + 4096 * wave + 1024 * j), 16,
                                                 b_goff[j], 0, 0, 0);
    };

    // Fragment reads (the transposing pattern of the kernel above, with the
    // wave's m block for A and its n block for B): fragment f, k half s:
    // lane (q, j16) points at k row 16s + 8*(q/2) + j16/4 (and 4 rows on for
    // the second read), columns 32f + 16*(q%2) + 4*(j16%4) .. +3 of the wave's
    // 128-column block.
    const int l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, j16 = lane & 15;
    const int brow = 8 * (q >> 1) + (j16 >> 2);
    const int bx = 2 * (q & 1) + ((j16 & 3) >> 1);
    const int bsw = (j16 >> 3) & 1;
    uint32_t fa_off[2], fb_off[2];
#pragma unroll
    for (int fp = 0; fp < 2; ++fp) {
        const uint32_t in_block = (uint32_t)(brow * 128 + 16 * (bx + 4 * (fp ^ bsw)) + 8 * (j16 & 1));
        fa_off[fp] = (uint32_t)(wm * 2 * 4096) + in_block;
        fb_off[fp] = (uint32_t)(wn * 2 * 4096) + in_block;
    }
    auto tr_read = [&](const char *stage, uint32_t off) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + off));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + off + 512));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 fa[2][4], fb[2][4];
    // Read slot r (0..7) of half s of the slice in stage si into register set
    // `set`, in the order the next block of matrix instructions consumes them:
    // A0, B0, B1, B2, B3, A1, A2, A3.
    auto read_slot = [&](int si, int s, int set, int r) {
        if (r == 0 || r >= 5) {
            const int f = r == 0 ? 0 : r - 4;
            fa[set][f] = tr_read(a_stage(si), fa_off[f & 1] + 4096 * (f >> 1) + 2048 * s);
        } else {
            const int f = r - 1;
            fb[set][f] = tr_read(b_stage(si), fb_off[f & 1] + 4096 * (f >> 1) + 2048 * s);
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    auto mma = [&](int set, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Prologue: slices 0..2 whole and loads 0, 1 of slice 3, A before B in
    // each; slice 0 is followed by 20 loads.
    const int nk = (K + BK - 1) / BK;
    {
        const rsrc_t ra0 = rsrc_a(0), ra1 = rsrc_a(1), ra2 = rsrc_a(2), ra3 = rsrc_a(3);
        const rsrc_t rb0 = rsrc_b(0), rb1 = rsrc_b(1), rb2 = rsrc_b(2), rb3 = rsrc_b(3);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(0, ra0, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(0, rb0, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(1, ra1, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(1, rb1, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_a(2, ra2, j);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_b(2, rb2, j);
        dma_a(3, ra3, 0);
        dma_a(3, ra3, 1);
        dma_b(3, rb3, 0);
        dma_b(3, rb3, 1);
    }
    rsrc_t ra_pend = rsrc_a(3), rb_pend = rsrc_b(3);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(20));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 8; ++r) read_slot(0, 0, 0, r);
    auto slice = [&](int u, int kt) {
        const int st = u % 4, st3 = (u + 3) % 4, st_n = (u + 1) % 4;
        rsrc_t ra_next, rb_next;
        // Block 1: the slice's first k half; reads of its second half; loads
        // 2, 3 of slice kt + 3.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            mma(0, t);
            if (t < 8) read_slot(st, 1, 1, t);
            else if (t == 9) dma_a(st3, ra_pend, 2);
            else if (t == 11) dma_b(st3, rb_pend, 2);
            else if (t == 13) dma_a(st3, ra_pend, 3);
            else if (t == 15) dma_b(st3, rb_pend, 3);
            else if (t == 8) ra_next = rsrc_a(kt + 4);
            else if (t == 10) rb_next = rsrc_b(kt + 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(16));
        __builtin_amdgcn_s_barrier();
        // Block 2: the second k half while the first half of slice kt + 1 is
        // read; loads 0, 1 of slice kt + 4 into this slice's stages.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            mma(1, t);
            if (t & 1) read_slot(st_n, 0, 0, t >> 1);
            else if (t == 0) dma_a(st, ra_next, 0);
            else if (t == 2) dma_b(st, rb_next, 0);
            else if (t == 4) dma_a(st, ra_next, 1);
            else if (t == 6) dma_b(st, rb_next, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        ra_pend = ra_next;
        rb_pend = rb_next;
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

    // Each wave's 32 KB of staging: two consecutive stages.
    char *lo = wave == 0 ? sa0 : wave == 1 ? sa2 : wave == 2 ? sb0 : sb2;
    char *hi = wave == 0 ? sa1 : wave == 1 ? sa3 : wave == 2 ? sb1 : sb3;
    lines_epilogue<OUT, false>(p, acc, [&](int row) -> char * {
        return (row < 64 ? lo : hi) + (row & 63) * 256;
    }, m0, n0, wm, wn, lane);
}

// The kernel above at 128 x 128 (each wave 64 x 64): four 8 KB single-slice
// stages per operand (two 64-column blocks of 32 k rows), 64 KB in all.
// Every block of 4 matrix instructions issues one load of A and one of B:
// slice s's load 0 in block 2 of slice s - 4, load 1 in block 1 of slice s
// - 3, so 8 loads per lane follow the last one slice kt + 1 needs by the
// barrier of slice kt.  Same bits as the 256 x 256 kernel.
template <int OUT>
__global__ void __launch_bounds__(256)
bf16_lines128_tn_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 128, BN = 128, BK = 32;
    constexpr int kSlice = BK * 128 * 2;      // 8 KB: 32 k rows x 128 columns
    constexpr int UNROLL = 4;
    __shared__ __attribute__((aligned(1024))) char sa0[kSlice], sa1[kSlice], sa2[kSlice], sa3[kSlice];
    __shared__ __attribute__((aligned(1024))) char sb0[kSlice], sb1[kSlice], sb2[kSlice], sb3[kSlice];
    auto a_stage = [&](int i) -> char * { return i == 0 ? sa0 : i == 1 ? sa1 : i == 2 ? sa2 : sa3; };
    auto b_stage = [&](int i) -> char * { return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : sb3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, 4, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);

    // Load j (0..1) of a slice, for either operand: g = 2*wave + j covers
    // block g/4 (columns 64*(g/4) ..), k rows 8*(g%4) .. +7 (lane -> k row
    // 8*(g%4) + lane/8, physical chunk lane%8), landing at stage + 1024 g.
    uint32_t a_goff[2], b_goff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int g = 2 * wave + j;
        const int row = 8 * (g & 3) + (lane >> 3);
        const int lc = (lane & 7) ^ lines_swz_b(row);
        a_goff[j] = (uint32_t)(row * lda + 64 * (g >> 2) + 8 * lc) * 2u;
        b_goff[j] = (uint32_t)(row * ldb + 64 * (g >> 2) + 8 * lc) * 2u;
    }
    auto rsrc_a = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent(((int64_t)(K - k0 - 1) * lda + (M - m0)) * 2));
    };
    auto rsrc_b = [&](int s) {
        const int k0 = BK * s;
        return make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
    };
    auto dma_a = [&](int si, const rsrc_t &ra, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(a_stage(si) + 1024 * (2 * wave + j)), 16,
                                                 a_goff[j], 0, 0, 0);
    };
    auto dma_b = [&](int si, const rsrc_t &rb, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(b_stage(si) + 1024 * (2 * wave + j)), 16,
                                                 b_goff[j], 0, 0, 0);
    };

    // Fragment f, k half s of the wave's 64-column block (m for A, n for B):
    // the transposing reads of the kernel above.
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, j16 = lane & 15;
    const int brow = 8 * (q >> 1) + (j16 >> 2);
    const int bx = 2 * (q & 1) + ((j16 & 3) >> 1);
    const int bsw = (j16 >> 3) & 1;
    uint32_t fa_off[2], fb_off[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const uint32_t in_block = (uint32_t)(brow * 128 + 16 * (bx + 4 * (f ^ bsw)) + 8 * (j16 & 1));
        fa_off[f] = (uint32_t)(wm * 4096) + in_block;
        fb_off[f] = (uint32_t)(wn * 4096) + in_block;
    }
    auto tr_read = [&](const char *stage, uint32_t off) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + off));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(stage + off + 512));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 fa[2][2], fb[2][2];
    // Read slot r (0..3): A0, B0, B1, A1.
    auto read_slot = [&](int si, int s, int set, int r) {
        if (r == 0 || r == 3) {
            const int f = r == 0 ? 0 : 1;
            fa[set][f] = tr_read(a_stage(si), fa_off[f] + 2048 * s);
        } else {
            fb[set][r - 1] = tr_read(b_stage(si), fb_off[r - 1] + 2048 * s);
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    auto mma = [&](int set, int t) {
        const int i = t >> 1, j = t & 1;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Prologue: slices 0..2 whole and load 0 of slice 3, A before B in each;
    // slice 0 is followed by 10 loads.
    const int nk = (K + BK - 1) / BK;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
        const rsrc_t ra = rsrc_a(s2), rb = rsrc_b(s2);
#pragma unroll
        for (int j = 0; j < (s2 < 3 ? 2 : 1); ++j) dma_a(s2, ra, j);
#pragma unroll
        for (int j = 0; j < (s2 < 3 ? 2 : 1); ++j) dma_b(s2, rb, j);
    }
    rsrc_t ra_pend = rsrc_a(3), rb_pend = rsrc_b(3);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(10));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 4; ++r) read_slot(0, 0, 0, r);
    auto slice = [&](int u, int kt) {
        const int st = u % 4, st3 = (u + 3) % 4, st_n = (u + 1) % 4;
        rsrc_t ra_next, rb_next;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            mma(0, t);
            read_slot(st, 1, 1, t);
            if (t == 0) ra_next = rsrc_a(kt + 4);
            else if (t == 1) dma_a(st3, ra_pend, 1);
            else if (t == 2) rb_next = rsrc_b(kt + 4);
            else dma_b(st3, rb_pend, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            mma(1, t);
            read_slot(st_n, 0, 0, t);
            if (t == 0) dma_a(st, ra_next, 0);
            else if (t == 2) dma_b(st, rb_next, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        ra_pend = ra_next;
        rb_pend = rb_next;
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

    // Each wave's 16 KB of staging: two consecutive stages.
    char *lo = wave == 0 ? sa0 : wave == 1 ? sa2 : wave == 2 ? sb0 : sb2;
    char *hi = wave == 0 ? sa1 : wave == 1 ? sa3 : wave == 2 ? sb1 : sb3;
    lines_epilogue<OUT, false>(p, acc, [&](int row) -> char * {
        return (row < 32 ? lo : hi) + (row & 31) * 256;
    }, m0, n0, wm, wn, lane);
}

hipError_t launch_bf16_lines128_tn(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 127) / 128, tiles_n = (p.N + 127) / 128;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&bf16_lines128_tn_kernel<GEMM_OUT_BF16>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&bf16_lines128_tn_kernel<GEMM_OUT_FP8>)
                                           : reinterpret_cast<const void *>(&bf16_lines128_tn_kernel<GEMM_OUT_F32>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

hipError_t launch_bf16_lines_tn(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&bf16_lines_tn_kernel<GEMM_OUT_BF16>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&bf16_lines_tn_kernel<GEMM_OUT_FP8>)
                                           : reinterpret_cast<const void *>(&bf16_lines_tn_kernel<GEMM_OUT_F32>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

template <bool BT>
hipError_t launch_bf16_lines(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&bf16_lines_kernel<GEMM_OUT_BF16, BT>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&bf16_lines_kernel<GEMM_OUT_FP8, BT>)
                                           : reinterpret_cast<const void *>(&bf16_lines_kernel<GEMM_OUT_F32, BT>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

template <bool BT>
hipError_t launch_bf16_lines128(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 127) / 128, tiles_n = (p.N + 127) / 128;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn = out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&bf16_lines128_kernel<GEMM_OUT_BF16, BT>)
                     : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&bf16_lines128_kernel<GEMM_OUT_FP8, BT>)
                                           : reinterpret_cast<const void *>(&bf16_lines128_kernel<GEMM_OUT_F32, BT>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

template __global__ void bf16_lines_kernel<GEMM_OUT_F32, false>(GemmParams, int, int);
template __global__ void bf16_lines_kernel<GEMM_OUT_BF16, false>(GemmParams, int, int);
template __global__ void bf16_lines_kernel<GEMM_OUT_FP8, false>(GemmParams, int, int);
template __global__ void bf16_lines_kernel<GEMM_OUT_F32, true>(GemmParams, int, int);
template __global__ void bf16_lines_kernel<GEMM_OUT_BF16, true>(GemmParams, int, int);
template __global__ void bf16_lines_kernel<GEMM_OUT_FP8, true>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_F32, false>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_BF16, false>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_FP8, false>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_F32, true>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_BF16, true>(GemmParams, int, int);
template __global__ void bf16_lines128_kernel<GEMM_OUT_FP8, true>(GemmParams, int, int);
template __global__ void bf16_lines_tn_kernel<GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_lines128_tn_kernel<GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_lines128_tn_kernel<GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_lines128_tn_kernel<GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_lines_tn_kernel<GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_lines_tn_kernel<GEMM_OUT_FP8>(GemmParams, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
const KernelDesc kBf16LinesKernels[] = {
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 64, 256, 8, 8, "bf16_mfma32_256x256x64_w2x2_a8b8_lines",
     &launch_bf16_lines<false>, 1024, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 64, 256, 8, 8, "bf16_mfma32_256x256x64_w2x2_a8b8_nt_lines",
     &launch_bf16_lines<true>, 1024, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_tn_lines",
     &launch_bf16_lines_tn, 1024, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 128, 128, 64, 256, 8, 8, "bf16_mfma32_128x128x64_w2x2_a8b8_lines",
     &launch_bf16_lines128<false>, 256, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 128, 128, 64, 256, 8, 8, "bf16_mfma32_128x128x64_w2x2_a8b8_nt_lines",
     &launch_bf16_lines128<true>, 256, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 128, 128, 32, 256, 8, 8, "bf16_mfma32_128x128x32_w2x2_a8b8_tn_lines",
     &launch_bf16_lines128_tn, 256, nullptr, kLayoutTN, false, kOutAll},
};
const int kBf16LinesKernelCount = sizeof(kBf16LinesKernels) / sizeof(kBf16LinesKernels[0]);
#endif

}  // namespace gemm
