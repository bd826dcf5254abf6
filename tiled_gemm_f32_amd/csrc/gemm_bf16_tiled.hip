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

// Physical chunk of logical chunk `ch` in LDS row `row` (rows are 128 bytes).
// With this XOR the three access patterns below touch distinct 16-byte bank
// slots in every group of 8 lanes (a 128-byte bank window) and of 16 lanes
// (a 256-byte window): fragment reads (32 consecutive rows, one chunk),
// A-panel writes (8 lanes per row, all chunks) and the transposed B writes
// (one row per lane, 8 rows apart, with the column parity flipped for lanes
// 8-15 of each group of 16; see stash_b).
__device__ __forceinline__ int swz(int row, int ch) { return ch ^ (row & 7) ^ ((row >> 3) & 7); }

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
__global__ void __launch_bounds__(64 * WM * WN)
bf16_tiled_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
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
        a_off[i] = panel_off(r, a_rows, lda, ch * 8, 2);
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

    auto stash_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Cfg::kAPer; ++i) lds_a[buf][a_lds[i]] = sa[i];
    };
    auto stash_b = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Cfg::kBPer; ++i) {
            // sb[i][e] word w holds columns (2w, 2w+1) of k row e.  Column c of
            // the transposed block needs, in word q, rows (2q, 2q+1) of column c.
            // Write number c of a lane stores column c ^ flip, flip = bit 3 of
            // its block column: lanes 8-15 of each 16 then write the opposite
            // row parity, which keeps the 16 stores on distinct bank slots.
            const uint32_t flip = (b_ng[i] >> 3) & 1;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint32_t w[KR / 2];
#pragma unroll
                for (int q = 0; q < KR / 2; ++q) {
                    const uint32_t lo = sb[i][2 * q][c >> 1], hi = sb[i][2 * q + 1][c >> 1];
                    const uint32_t even = (lo & 0xffffu) | (hi << 16);
                    const uint32_t odd = (lo >> 16) | (hi & 0xffff0000u);
                    w[q] = ((c & 1) ^ flip) ? odd : even;
                }
                const int row = 8 * b_ng[i] + (c ^ (int)flip);
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

    // Two fragment register sets: step s+1 is read from LDS while the
    // matrix cores work on step s.
    bf16x8 fa[2][Cfg::kFragM], fb[2][Cfg::kFragN];
    auto read_frags = [&](int buf, int s, int set) {
        // Lane (row l32, half h) supplies k = 16*s + 8*h .. 16*s + 8*h + 7.
        const int ch = 2 * s + h;
#pragma unroll
        for (int fm = 0; fm < Cfg::kFragM; ++fm) {
            const int row = wm * Cfg::kWaveM + 32 * fm + l32;
            fa[set][fm] = __builtin_bit_cast(bf16x8, lds_a[buf][row * Cfg::kChunks + swz(row, ch)]);
        }
#pragma unroll
        for (int fn = 0; fn < Cfg::kFragN; ++fn) {
            const int row = wn * Cfg::kWaveN + 32 * fn + l32;
            fb[set][fn] = __builtin_bit_cast(bf16x8, lds_b[buf][row * Cfg::kChunks + swz(row, ch)]);
        }
    };
    auto mfmas = [&](int set) {
#pragma unroll
        for (int fm = 0; fm < Cfg::kFragM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::kFragN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][fm], fb[set][fn], acc[fm][fn], 0, 0, 0);
    };

    // Pipeline.  At the top of iteration kt, LDS buffer kt&1 holds slice kt
    // (step 0 already in registers) and the staging registers hold slice
    // kt+1.  During the k-steps of slice kt the staging registers are written
    // to the other LDS buffer and refilled with slice kt+2, so global latency
    // is covered by most of a slice of matrix work.  The body is straight-line:
    // slices past the end read as zero through the buffer extents and land in
    // a buffer that is never read again.
    constexpr int kStashA = Cfg::kSteps > 1 ? 1 : 0;
    constexpr int kStashB = Cfg::kSteps > 2 ? 2 : Cfg::kSteps - 1;
    const int nk = (K + BK - 1) / BK;
    fetch(0);
    stash_a(0);
    stash_b(0);
    __syncthreads();
    fetch(1);
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
#pragma unroll
        for (int s = 0; s < Cfg::kSteps; ++s) {
            if (s + 1 < Cfg::kSteps) read_frags(cur, s + 1, (s + 1) & 1);
            mfmas(s & 1);
            if (s == kStashA) stash_a(cur ^ 1);
            if (s == kStashB) {
                stash_b(cur ^ 1);
                fetch(kt + 2);
            }
        }
        __syncthreads();
        read_frags(cur ^ 1, 0, 0);
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

// ---------------------------------------------------------------------------
// Pipelined kernel for the common case: 256 x 256 x 64 workgroup tile, four
// waves of 128 x 128, 16-byte loads of both operands (aligned A and B whose
// leading dimensions and K, N are multiples of 8).  Same data layout and
// numerics as the generic kernel above; the difference is instruction count
// per slice, which decides how densely one wave per SIMD can issue MFMAs:
//   * every LDS address is a per-lane base register plus an immediate (the
//     swizzle factors into a lane constant XOR compile-time step bits, and
//     the slice loop is unrolled twice so the buffer is a constant);
//   * global loads use constant per-lane offsets against buffer resources
//     rebased each slice with scalar arithmetic;
//   * the B transpose is one byte-permute per output word, the permute
//     selector absorbing the per-lane column-parity flip;
//   * the barrier sits after the last LDS store of a slice, so the first
//     fragment reads of the next slice overlap the last 16 MFMAs.
// ---------------------------------------------------------------------------
constexpr uint32_t kSelEven = 0x05040100u;   // low halves of (x, y) -> (x.lo, y.lo)
constexpr uint32_t kSelOdd = 0x07060302u;    // high halves of (x, y) -> (x.hi, y.hi)

template <int GROUP_M>
__global__ void __launch_bounds__(256)
bf16_pipe_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int kABuf = BM * BK * 2;          // bytes of one A panel (32 KB)
    constexpr int kBBuf = BN * BK * 2;          // bytes of one B panel (32 KB)
    constexpr int kBBase = 2 * kABuf;           // B panels follow both A panels
    __shared__ __attribute__((aligned(16))) char lds[2 * kABuf + 2 * kBBuf];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    const int a_rows = min(BM, M - m0);

    // Global loads.  A: chunk (row tid/8 + 32i, k chunk tid%8), i = 0..7.
    // B: block (k rows 8*(tid/32) + e, n columns 8*(tid%32) .. +7), e = 0..7.
    const int a_ch = tid & 7, a_r0 = tid >> 3;
    const int b_kg = tid >> 5, b_ng = tid & 31;
    uint32_t a_off[8], b_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a_off[i] = panel_off(a_r0 + 32 * i, a_rows, lda, 8 * a_ch, 2);
        b_off[i] = (uint32_t)((8 * b_kg + i) * ldb + 8 * b_ng) * 2u;
    }
    u32x4 ga[8], gb[8];
    auto fetch = [&](int kt) {
        const int k0 = kt * BK;
        // Rebased per slice: rows past K fall outside the extents, rows past M
        // read row M - 1, and a chunk at or past K in a row of A is forced out
        // of range.
        const rsrc_t ra = make_rsrc(A + (int64_t)m0 * lda + k0,
                                    clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 2));
        const rsrc_t rb = make_rsrc(B + (int64_t)k0 * ldb + n0,
                                    clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
        // Offsets stay below 2^31, so adding 2^31 lands every load of an
        // out-of-range chunk outside the extent (arithmetic rather than a
        // select, which the compiler would turn into divergent branches).
        const uint32_t poison = (uint32_t)(8 * a_ch >= K - k0) << 31;
#pragma unroll
        for (int i = 0; i < 8; ++i) ga[i] = load_b128(ra, a_off[i] + poison);
#pragma unroll
        for (int e = 0; e < 8; ++e) gb[e] = load_b128(rb, b_off[e]);
    };

    // LDS write addresses.  Physical chunk = logical ^ (row & 7) ^ ((row >> 3) & 7)
    // (same swizzle as swz()), folded into per-lane bases.
    const int a_p = a_ch ^ (a_r0 & 7) ^ wave;                   // (row >> 3) & 7 = wave ^ 4*(i & 1)
    const uint32_t a_w0 = (uint32_t)(a_r0 * 128 + 16 * a_p);
    const uint32_t a_w1 = (uint32_t)(a_r0 * 128 + 16 * (a_p ^ 4));
    const uint32_t flip = (uint32_t)(b_ng >> 3) & 1u;           // see the generic kernel's stash_b
    uint32_t b_w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int col = c ^ (int)flip;
        b_w[c] = (uint32_t)(kBBase + 128 * (8 * b_ng + col) + 16 * (b_kg ^ col ^ (b_ng & 7)));
    }
    const uint32_t sel_even_c = flip ? kSelOdd : kSelEven;     // selector for writes c = 0, 2, 4, 6
    const uint32_t sel_odd_c = flip ? kSelEven : kSelOdd;      // and for c = 1, 3, 5, 7

    auto stash_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4 *>(lds + ((i & 1) ? a_w1 : a_w0) + 4096 * i + buf * kABuf) = ga[i];
    };
    auto stash_b = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t sel = (c & 1) ? sel_odd_c : sel_even_c;
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = __builtin_amdgcn_perm(gb[2 * q + 1][c >> 1], gb[2 * q][c >> 1], sel);
            *reinterpret_cast<u32x4 *>(lds + b_w[c] + buf * kBBuf) = v;
        }
    };

    // Fragment read bases: row = w*128 + 32*f + l32, logical chunk 2s + h.
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int y = (l32 & 7) ^ (l32 >> 3) ^ h;
    uint32_t ra_t[4], rb_t[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ra_t[t] = (uint32_t)((wm * 128 + l32) * 128 + 16 * (y ^ (2 * t)));
        rb_t[t] = (uint32_t)(kBBase + (wn * 128 + l32) * 128 + 16 * (y ^ (2 * t)));
    }
    bf16x8 fa[2][4], fb[2][4];
    auto read_frags = [&](int buf, int s, int set) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int t = s ^ (2 * (f & 1));
            fa[set][f] = *reinterpret_cast<const bf16x8 *>(lds + ra_t[t] + 4096 * f + buf * kABuf);
            fb[set][f] = *reinterpret_cast<const bf16x8 *>(lds + rb_t[t] + 4096 * f + buf * kBBuf);
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    auto mfmas = [&](int set) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    };
    // One slice.  Slices past the end read as zero and change nothing, so
    // the loop below may run one slice beyond an odd count.
    auto slice = [&](int kt, int cur) {
        read_frags(cur, 1, 1);
        mfmas(0);
        read_frags(cur, 2, 0);
        mfmas(1);
        stash_a(cur ^ 1);
        read_frags(cur, 3, 1);
        mfmas(0);
        stash_b(cur ^ 1);
        fetch(kt + 2);
        __syncthreads();
        read_frags(cur ^ 1, 0, 0);
        mfmas(1);
    };

    const int nk = (K + BK - 1) / BK;
    fetch(0);
    stash_a(0);
    stash_b(0);
    __syncthreads();
    fetch(1);
    read_frags(0, 0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
        slice(kt, 0);
        slice(kt + 1, 1);
    }

    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
            const int col = n0 + wn * 128 + 32 * fn + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + 32 * fm + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) {
                    float *cp = p.C + (int64_t)row * p.ldc + col;
                    float v = alpha * acc[fm][fn][r];
                    if (beta != 0.0f) v = fmaf(beta, *cp, v);
                    *cp = epilogue_value(v, col, p.bias, p.act);
                }
            }
        }
    }
}

template <int GROUP_M>
hipError_t launch_bf16_pipe(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&bf16_pipe_kernel<GROUP_M>),
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0, stream);
}

// ---------------------------------------------------------------------------
// Ring kernel: the gfx950-native form of the double-buffered pipeline.
//
// A k-slice of a 256 x 256 tile needs 32 KB of operands per 1024 MFMA cycles
// (BK = 32), and a slice that misses L2 takes several microseconds to arrive.
// Register staging cannot hold several slices in flight, so both panels are
// copied straight from HBM into an LDS ring of NS slices with
// buffer_load ... lds (lane i of a wave instruction lands at LDS base +
// 16*i; the lane chooses which global 16 bytes to fetch, which is how the
// layouts below are swizzled).  Slice kt+NS is requested as soon as slice kt
// has been consumed, so each load has NS-1 slices of MFMA work to arrive
// (the multi-buffered pipelining of "What is left", carried to NS stages).
//
//   A slice: [256 rows][4 chunks of 16 B], chunk ^= (row >> 2) & 3.
//     Fragment reads are 16-byte ds_read_b128 (k contiguous per row).
//   B slice: 8 blocks of 32 columns, each [32 k][64 B] (row-major as in HBM),
//     16-byte chunk ^= 2 * ((k >> 1) & 1).  Fragments come from the
//     transposing ds_read_b64_tr_b16: in each group of 16 lanes, lane s
//     points at k row k0 + s/4, columns c0 + 4*(s%4) .. +3, and lane j
//     receives column c0 + j of rows k0 .. k0+3 -- the B operand layout of
//     the matrix instruction, with no register transpose.
// Bank behaviour, as measured with the LDS conflict counters on gfx950: a
// ds_read_b128 is served in two halves of 32 lanes, each costing as many
// cycles as its most-loaded 4-byte bank (64 banks, 256-byte period), and
// some lane pairings cost extra beyond that model (the earlier swizzle
// ((row >> 1) ^ (row >> 3)) & 3, conflict-free on paper, measured twice the
// cycles).  (row >> 2) & 3 measured conflict-free, as did the B reads and the
// contiguous DMA writes.
// ---------------------------------------------------------------------------


__device__ __forceinline__ int ring_swz_a(int row) { return (row >> 2) & 3; }

// BT: B is stored transposed (N x K, k contiguous), so its slices take the A
// layout, loads and fragment reads above, and N needs no alignment: runs of
// C columns that straddle N are stored element by element.
// AT: A is stored transposed (K x M, m contiguous), the shape of an
// untransposed B, so its slices take the B layout, loads and transposing
// reads above.  The reads deliver each lane's k values in the same order as
// the 16-byte reads do, so either form of A pairs with either form of B.
template <int NS, int GROUP_M, bool BT, bool AT, int OUT>
__global__ void __launch_bounds__(256)
bf16_ring_kernel(GemmParams p, int tiles_m, int tiles_n) {
    apply_k_split<uint16_t>(p);
    constexpr int BM = 256, BN = 256, BK = 32;
    constexpr int kA = BM * BK * 2;     // 16 KB of A per slice
    constexpr int kB = BN * BK * 2;     // 16 KB of B per slice
    constexpr int kStage = kA + kB;
    // One array per stage: with distinct objects the compiler can tell that
    // fragment reads of one stage do not depend on DMA still landing in
    // another, and does not wait for the whole ring.
    __shared__ __attribute__((aligned(1024))) char st0[kStage], st1[kStage], st2[kStage], st3[kStage],
        st4[NS > 4 ? kStage : 16];
    auto stage_base = [&](int st) -> char * {
        return st == 0 ? st0 : st == 1 ? st1 : st == 2 ? st2 : st == 3 ? st3 : st4;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords_square(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);

    // DMA instruction j of this wave fills 1 KB block 4*wave + j of each panel.
    //   A block: rows 16*blk .. +15; lane -> row 16*blk + lane/4, physical chunk lane%4.
    //   B block: column block blk/2, k rows 16*(blk&1) .. +15; lane -> k row 16*(blk&1) + lane/4.
    uint32_t a_goff[4], b_goff[4];
    int a_kc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int blk = 4 * wave + j;
        const int ra = 16 * blk + (lane >> 2);
        const int lca = (lane & 3) ^ ring_swz_a(ra);
        a_kc[j] = 8 * lca;
        a_goff[j] = panel_off(ra, a_rows, lda, 8 * lca, 2);
        if (AT) {
            // Rows of A^T (k rows, m contiguous) laid out as an untransposed B.
            const int mb = blk >> 1, rk = 16 * (blk & 1) + (lane >> 2);
            const int lck = (lane & 3) ^ (2 * ((rk >> 1) & 1));
            a_goff[j] = (uint32_t)(rk * lda + 32 * mb + 8 * lck) * 2u;
        }
        if (BT) {
            // Rows of B^T (columns of B) laid out as A's rows; same chunk k as A.
            b_goff[j] = panel_off(ra, b_rows, ldb, 8 * lca, 2);
        } else {
            const int nb = blk >> 1, rb = 16 * (blk & 1) + (lane >> 2);
            const int lcb = (lane & 3) ^ (2 * ((rb >> 1) & 1));
            b_goff[j] = (uint32_t)(rb * ldb + 32 * nb + 8 * lcb) * 2u;
        }
    }
    // Resources of slice kt.  Rebased per slice: k rows past K fall outside
    // the extents, rows past M (past N for B^T) read the last valid row, and a
    // chunk at or past K in a row of A (or B^T) gets 2^31 added to its offset.
    auto slice_rsrc = [&](int kt, rsrc_t &ra, rsrc_t &rb) {
        const int k0 = kt * BK;
        if (AT)
            ra = make_rsrc(A + (int64_t)k0 * lda + m0, clamp_extent(((int64_t)(K - k0 - 1) * lda + (M - m0)) * 2));
        else
            ra = make_rsrc(A + (int64_t)m0 * lda + k0, clamp_extent(((int64_t)(a_rows - 1) * lda + (K - k0)) * 2));
        if (BT)
            rb = make_rsrc(B + (int64_t)n0 * ldb + k0, clamp_extent(((int64_t)(b_rows - 1) * ldb + (K - k0)) * 2));
        else
            rb = make_rsrc(B + (int64_t)k0 * ldb + n0, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 2));
    };
    // DMA instruction j (0..7) of slice kt into `stage`: j < 4 fills A block
    // 4*wave + j, j >= 4 fills B block 4*wave + j - 4.
    auto dma = [&](int kt, int stage, const rsrc_t &ra, const rsrc_t &rb, int j) {
        if (j < 4) {
            // (A^T rows past K already fall outside the extent.)
            const uint32_t poison = AT ? 0u : (uint32_t)(a_kc[j] >= K - kt * BK) << 31;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void *)(stage_base(stage) + (4 * wave + j) * 1024), 16, a_goff[j] + poison, 0, 0, 0);
        } else {
            // B^T chunks past K in a valid row would read the next row: poison them as A's.
            const uint32_t poison = BT ? (uint32_t)(a_kc[j - 4] >= K - kt * BK) << 31 : 0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void *)(stage_base(stage) + kA + (4 * wave + j - 4) * 1024), 16, b_goff[j - 4] + poison,
                0, 0, 0);
        }
    };
    // Fragment read bases (bytes within a slice).
    const int h = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    uint32_t fa_base[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        fa_base[s] = (uint32_t)((wm * 128 + l32) * 64 + 16 * ((2 * s + h) ^ ring_swz_a(l32)));
    const int q = lane >> 4, j16 = lane & 15;
    const int brow = 8 * (q >> 1) + (j16 >> 2);
    const int bch = 2 * (q & 1) + ((j16 & 3) >> 1);
    const uint32_t fb_base = (uint32_t)(kA + wn * 4 * 2048 + brow * 64 + 16 * (bch ^ (2 * ((brow >> 1) & 1))) +
                                        8 * (j16 & 1));
    // AT: A^T fragment reads, the transposing pattern of B in the A half of the stage.
    const uint32_t fat_base = (uint32_t)(wm * 4 * 2048 + brow * 64 + 16 * (bch ^ (2 * ((brow >> 1) & 1))) +
                                         8 * (j16 & 1));
    uint32_t fbt_base[2];   // BT: B^T fragment reads, the A pattern in the B half of the stage
#pragma unroll
    for (int s = 0; s < 2; ++s)
        fbt_base[s] = (uint32_t)(kA + (wn * 128 + l32) * 64 + 16 * ((2 * s + h) ^ ring_swz_a(l32)));

    bf16x8 fa[2][4], fb[2][4];
    // Fragment read slot r (0..7) of half s of the slice in `stage` into
    // register set `set`, in the order the next MFMA block consumes them:
    // A0, B0, B1, B2, B3, A1, A2, A3 (one ds_read_b128, or two
    // ds_read_b64_tr_b16 for a B fragment).
    auto read_slot = [&](int stage, int s, int set, int r) {
        char *base = stage_base(stage);
        if ((r == 0 || r >= 5) && AT) {
            const int f = r == 0 ? 0 : r - 4;
            const int aoff = fat_base + 2048 * f + 1024 * s;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + aoff));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + aoff + 256));
            fa[set][f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else if (r == 0 || r >= 5) {
            const int f = r == 0 ? 0 : r - 4;
            fa[set][f] = *reinterpret_cast<const bf16x8 *>(base + fa_base[s] + 2048 * f);
        } else if (BT) {
            const int f = r - 1;
            fb[set][f] = *reinterpret_cast<const bf16x8 *>(base + fbt_base[s] + 2048 * f);
        } else {
            const int f = r - 1;
            const int boff = fb_base + 2048 * f + 1024 * s;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + boff));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + boff + 256));
            fb[set][f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    // The matrix core is given B^T as its first operand and A^T as its
    // second, so it accumulates the transposed tile (C^T = B^T A^T): each
    // lane then holds runs of 4 consecutive columns of one row of C, which
    // the epilogue writes with 16-byte stores.
    auto mma = [&](int set, int t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
    };

    // Slice kt lives in stage kt % NS.  Each slice is two blocks of 16
    // MFMAs.  Block 1 multiplies the first k half (register set 0) while the
    // second half is read into set 1; then every wave waits for slice kt+1
    // to land and for all reads of stage kt % NS to finish (barrier), and
    // block 2 multiplies set 1 while refilling that stage with slice kt+NS
    // and reading the first half of slice kt+1 into set 0.  The other
    // instructions are placed one per MFMA and pinned there with
    // sched_barrier, so the matrix pipe never waits on an LDS read that was
    // issued just before it.  Before the barrier of slice kt the only loads
    // allowed in flight are those of slices kt+2 .. kt+NS-1, 8 per lane each.
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
    for (int r = 0; r < 8; ++r) read_slot(0, 0, 0, r);
    for (int kb = 0; kb < nk; kb += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int kt = kb + u;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(0, t);
                if (t < 8) read_slot(u, 1, 1, t);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 * (NS - 2)));
            __builtin_amdgcn_s_barrier();
            rsrc_t ra, rb;
            slice_rsrc(kt + NS, ra, rb);      // zeros past the end
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                mma(1, t);
                if (t & 1) read_slot((u + 1) % NS, 0, 0, t >> 1);
                else dma(kt + NS, u, ra, rb, t >> 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Epilogue.  Register 4g + t of lane (h, l32) in fragment (fm, fn) is
    // C[row m0 + wm*128 + 32*fm + l32][column n0 + wn*128 + 32*fn + 8*g + 4*h + t].
    // Untransposed, N is a multiple of 8, so each run of 4 columns is wholly
    // inside or outside C; with B^T a run may straddle N and is then stored
    // element by element.  16-byte accesses need C 16-byte aligned and
    // ldc % 4 == 0.  The branch on the activation is taken once for the whole
    // tile, so each case is one fully unrolled pass and the accumulators stay
    // in registers.
    const float alpha = p.alpha, beta = p.beta;
    const bool vec_c = ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 4 == 0);
    with_activation(p.act, [&](auto act) {
        using Act = decltype(act);
        const bool vec_o = out_vec4<OUT>(p);
#pragma unroll
            for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * 128 + 32 * fn + 8 * g + 4 * h;
                    if (col >= N) continue;
                    // With B untransposed N is a multiple of 8, so a run of 4
                    // columns is never cut by N.
                    const bool whole = !BT || col + 4 <= N;
                    float b[4];   // -0.0 is the identity of IEEE addition, signed zeros included
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        b[t] = (p.bias != nullptr && (!BT || col + t < N)) ? p.bias[col + t] : -0.0f;
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
                        for (int t = 0; t < 4; ++t) v[t] = Act::apply(v[t] + b[t]);
                        if (whole)
                            store_out4<OUT>(p, row, col, v, vec_o);
                        else
                            store_out_first<OUT>(p, row, col, v, N - col);
                    }
                }
            }
    });
}

template <int NS, int GROUP_M, bool BT = false, bool AT = false>
hipError_t launch_bf16_ring(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + 255) / 256, tiles_n = (p.N + 255) / 256;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    const int out = launch_out_type(p);
    const void *fn =
        out == GEMM_OUT_BF16  ? reinterpret_cast<const void *>(&bf16_ring_kernel<NS, GROUP_M, BT, AT, GEMM_OUT_BF16>)
        : out == GEMM_OUT_FP8 ? reinterpret_cast<const void *>(&bf16_ring_kernel<NS, GROUP_M, BT, AT, GEMM_OUT_FP8>)
                              : reinterpret_cast<const void *>(&bf16_ring_kernel<NS, GROUP_M, BT, AT, GEMM_OUT_F32>);
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(256), argv, 0,
                           stream);
}

template <int BM, int BN, int BK, int WM, int WN, int VA, int VB, int GROUP_M>
hipError_t launch_bf16_tiled(const GemmParams &p, hipStream_t stream) {
    int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    GemmParams args = p;
    void *argv[] = {&args, (void *)&tiles_m, (void *)&tiles_n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&bf16_tiled_kernel<BM, BN, BK, WM, WN, VA, VB, GROUP_M>),
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)k_splits(p)), dim3(64 * WM * WN), argv, 0, stream);
}

#define BF16_TILED(BM, BN, BK, WM, WN, VA, VB, G)                                             \
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, BM, BN, BK, 64 * WM * WN, VA, VB,                   \
     "bf16_mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_a" #VA "b" #VB,                    \
     &launch_bf16_tiled<BM, BN, BK, WM, WN, VA, VB, G>, 0, nullptr, kLayoutNN, false,               \
     quantising_epilogue((BM / WM) * (BN / WN) / 64) ? kOutAll : kOutF32}

// Explicit instantiations: the device pass never sees the host-only table
// below, so the kernels it needs are named here.
template __global__ void bf16_pipe_kernel<4>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, false, GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, false, GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, false, GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<5, 4, false, false, GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<5, 4, false, false, GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<5, 4, false, false, GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, false, GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, false, GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, false, GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, true, GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, true, GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, false, true, GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, true, GEMM_OUT_F32>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, true, GEMM_OUT_BF16>(GemmParams, int, int);
template __global__ void bf16_ring_kernel<4, 4, true, true, GEMM_OUT_FP8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 8, 8, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<256, 256, 64, 2, 2, 1, 8, 4>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 8, 8, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 8, 1, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 1, 8, 8>(GemmParams, int, int);
template __global__ void bf16_tiled_kernel<128, 128, 64, 2, 2, 1, 1, 8>(GemmParams, int, int);

}  // namespace

// The table holds host function pointers, so it exists only in the host pass.
#if !defined(__HIP_DEVICE_COMPILE__)
const KernelDesc kBf16TiledKernels[] = {
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_ring4",
     &launch_bf16_ring<4, 4>, 1024, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_ring5",
     &launch_bf16_ring<5, 4>, 1024, nullptr, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 64, 256, 8, 8, "bf16_mfma32_256x256x64_w2x2_a8b8_pipe",
     &launch_bf16_pipe<4>},
    // Transposed layouts: the only fast kernels for them, so no K minimum.
    // vec_a / vec_b = 8: the stored rows of A and B are 16-byte multiples.
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_nt_ring4",
     &launch_bf16_ring<4, 4, true, false>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_tn_ring4",
     &launch_bf16_ring<4, 4, false, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_TILED, 256, 256, 32, 256, 8, 8, "bf16_mfma32_256x256x32_w2x2_a8b8_tt_ring4",
     &launch_bf16_ring<4, 4, true, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    // With B read element by element the 256 x 256 tile does not fit the
    // registers (its staged B values spill to scratch), so B without 16-byte
    // rows takes the 128 x 128 tiles below.
    BF16_TILED(256, 256, 64, 2, 2, 8, 8, 4),
    BF16_TILED(256, 256, 64, 2, 2, 1, 8, 4),
    BF16_TILED(128, 128, 64, 2, 2, 8, 8, 8),
    BF16_TILED(128, 128, 64, 2, 2, 8, 1, 8),
    BF16_TILED(128, 128, 64, 2, 2, 1, 8, 8),
    BF16_TILED(128, 128, 64, 2, 2, 1, 1, 8),
};
const int kBf16TiledKernelCount = sizeof(kBf16TiledKernels) / sizeof(kBf16TiledKernels[0]);
#endif

}  // namespace gemm
