// fp32 GEMM for skinny problems (M <= 16): the decode-GEMV case that
// "Tiled matrix multiplication" ("Avoid when") identifies as bandwidth-bound.
//
// With at most 16 rows of A, every element of B is used by at most 16
// multiply-adds, so the job is to stream B from HBM exactly once at full
// bandwidth while the matrix cores absorb the arithmetic:
//
//   * Each workgroup owns a strip of 16*VEC columns of C over the whole of
//     K, so B is read once in total.  Each lane loads VEC consecutive
//     columns of one k row (16 lanes cover the strip's row segment), four
//     k rows per wave instruction.
//   * The strip's k quads are dealt round-robin to the workgroup's waves,
//     each keeping UNROLL quads of loads in flight before consuming them, so
//     thousands of bytes are outstanding per wave.
//   * v_mfma_f32_16x16x4_f32 takes the 16 rows of A (lane row l%16, k row
//     l/16) against 16 columns of B; VEC instructions cover the lane's VEC
//     columns, column c of instruction j being strip column VEC*c + j.
//     Rows of A at or past M read as zero.  A may also be stored K x M
//     (transposed): its values then come from 4-byte loads of 4 rows of
//     the stored matrix.  A is 16 x K at most and is re-read from L2 by
//     every strip, so the narrower loads cost little next to B.
//   * The waves' partial 16 x (16*VEC) tiles are summed through LDS in a
//     fixed wave order (deterministic; no atomics) and the alpha/beta
//     epilogue is applied once per output.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

// B is streamed exactly once: non-temporal loads.
template <int V> struct BVec;
template <> struct BVec<4> {
    typedef f32x4 T;
    static __device__ __forceinline__ f32x4 load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(f32x4, load_b128_nt(r, off));
    }
};
template <> struct BVec<2> {
    typedef f32x2 T;
    static __device__ __forceinline__ f32x2 load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(f32x2, load_b64_nt(r, off));
    }
};
template <> struct BVec<1> {
    typedef float T;
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, load_b32_nt(r, off));
    }
};

template <int V, typename T> __device__ __forceinline__ float comp(const T &v, int j);
template <> __device__ __forceinline__ float comp<4, f32x4>(const f32x4 &v, int j) { return v[j]; }
template <> __device__ __forceinline__ float comp<2, f32x2>(const f32x2 &v, int j) { return v[j]; }
template <> __device__ __forceinline__ float comp<1, float>(const float &v, int) { return v; }

template <int VA> struct AVec;
template <> struct AVec<4> {
    // 16-byte load of k = 4*kq .. 4*kq+3 of the lane's row (whole vector in or out of range).
    static __device__ __forceinline__ f32x4 load(rsrc_t r, uint32_t off, int k, int K) {
        return __builtin_bit_cast(f32x4, load_b128(r, k < K ? off : kOutOfRange));
    }
};
template <> struct AVec<1> {
    static __device__ __forceinline__ f32x4 load(rsrc_t r, uint32_t off, int k, int K) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(float, load_b32(r, k + j < K ? off + 4u * j : kOutOfRange));
        return v;
    }
};

// The lane's A values of k block b: row lc, k = 16*b + 4*kq .. +3.  VA = 4
// or 1: A stored M x K (one 16-byte load, or four 4-byte ones, from
// a_base + 64*b).  VA = 0: A stored K x M (lda >= M), so the four k are
// four rows of the stored matrix and each value is one 4-byte load of
// column lc; a wave instruction reads 4 runs of 16 consecutive floats.
// Columns at or past M and k at or past K read as zero.
template <int VA>
__device__ __forceinline__ f32x4 load_a_quad(rsrc_t r, uint32_t a_base, int b, int kq, int lc, int K, int M,
                                             int lda) {
    const int k = 16 * b + 4 * kq;
    if constexpr (VA == 0) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_bit_cast(
                float, load_b32(r, lc < M && k + j < K ? (uint32_t)((k + j) * lda + lc) * 4u : kOutOfRange));
        return v;
    } else {
        return AVec<VA>::load(r, a_base + (uint32_t)b * 64u, k, K);
    }
}

// One workgroup per 16*VEC-column strip of C.  K is cut into 16-deep blocks,
// dealt round-robin to the waves.  Inside a block, lane group kq = lane/16
// owns k = 4*kq .. 4*kq+3 (one 16-byte load of its A row), and MFMA j of the
// block pairs k = 4*kq + j with B row 4*kq + j.  Blocks are processed in
// batches of UNROLL; the loads of batch t+1 are issued before batch t is
// consumed, so each wave always has a batch of loads in flight.
template <int VEC, int VA, int WAVES, int UNROLL>
__global__ void __launch_bounds__(64 * WAVES)
f32_skinny_kernel(GemmParams p) {
    constexpr int NW = 16 * VEC;
    typedef typename BVec<VEC>::T BT;
    __shared__ float red[WAVES][16][NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * NW;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kq = lane >> 4;     // k group within a 16-deep block
    const int lc = lane & 15;     // A row for the A operand; column group for B

    // A's extent ends after its last valid element (the host keeps it below
    // 2^31 bytes): rows at or past M read row M - 1, which only reaches rows
    // of C that are never stored, and k at or past K reads as zero.  B is
    // addressed through a resource rebased at the first k row of each batch
    // of loads, so offsets span one batch (at most 16*WAVES*UNROLL rows)
    // whatever the size of B; rows at or past K fall outside it and read as
    // zero.
    const rsrc_t ra = make_rsrc(p.A, clamp_extent((VA == 0 ? (int64_t)(K - 1) * lda + M : (int64_t)(M - 1) * lda + K) * 4));
    const float *b_strip = static_cast<const float *>(p.B) + n0;
    const uint32_t a_base = panel_off(lc, M, lda, 4 * kq, 4);
    const uint32_t b_base = (uint32_t)(4 * kq * ldb + VEC * lc) * 4u;
    const uint32_t b_row = (uint32_t)ldb * 4u;

    f32x4 acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = f32x4{};

    f32x4 av[2][UNROLL];
    BT bv[2][UNROLL][4];
    auto issue = [&](int set, int blk0) {
        const int k0 = 16 * blk0;
        const rsrc_t rb = make_rsrc(b_strip + (int64_t)k0 * ldb, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 4));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int b = blk0 + u * WAVES;
            av[set][u] = load_a_quad<VA>(ra, a_base, b, kq, lc, K, M, lda);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[set][u][j] = BVec<VEC>::load(rb, b_base + (uint32_t)(16 * u * WAVES + j) * b_row);
        }
    };
    auto consume = [&](int set) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < VEC; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[set][u][j], comp<VEC>(bv[set][u][j], c), acc[c], 0, 0, 0);
    };

    const int nb = (K + 15) >> 4;
    constexpr int kStride = WAVES * UNROLL;
    issue(0, wave);
    for (int blk0 = wave; blk0 < nb; blk0 += 2 * kStride) {
        issue(1, blk0 + kStride);        // past the end: reads zeros
        consume(0);
        issue(0, blk0 + 2 * kStride);
        consume(1);
    }

    // Register r of lane (kq, lc) is row 4*kq + r, column lc of its 16 x 16 block.
#pragma unroll
    for (int c = 0; c < VEC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * kq + r][VEC * lc + c] = acc[c][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    for (int idx = tid; idx < 16 * NW; idx += 64 * WAVES) {
        const int i = idx / NW, j = idx % NW;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][i][j];
        const int col = n0 + j;
        if (i < M && col < N) {
            float v = alpha * s;
            if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
            store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
        }
    }
}

// Single pass with A staged through LDS (A stored M x K, 16-byte aligned).
// The kernel above loads each lane's A values straight from memory: every
// wave instruction touches 16 rows of A 64 bytes at a time, lda apart, and
// since every strip re-reads all of A, those loads cost as much as a fifth
// of the call (the same kernel with A held constant in registers takes
// 47.6 us against 58.6 us at 16 x 8192 x 8192).  Here the workgroup loads
// the A chunk of a whole batch (16 rows x 16*WAVES*UNROLL k) with each
// wave instruction reading 1 KB of one row, stores it to LDS, and every wave
// reads its fragments from there.  Chunks are loaded two batches ahead into
// registers, written to one of three LDS buffers one batch ahead, and one
// barrier per batch orders the writes before the reads (the buffer written
// in batch t last held chunk t - 2, whose readers have all passed the
// barrier of batch t - 1).  Blocks, their k pairing and the order of the
// sums are those of f32_skinny_kernel, so the two give identical bits.
template <int VEC, int WAVES, int UNROLL>
__global__ void __launch_bounds__(64 * WAVES)
f32_skinny_lds_kernel(GemmParams p) {
    static_assert((16 * 16 * WAVES * UNROLL / 256) % WAVES == 0 && (16 * WAVES * UNROLL) % 256 == 0,
                  "the A chunk splits into whole 1 KB runs, the same number per wave");
    constexpr int NW = 16 * VEC;
    constexpr int kStride = WAVES * UNROLL;          // 16-deep blocks per batch
    constexpr int KC = 16 * kStride;                 // k per batch
    constexpr int ROW = KC + 4;                      // floats per LDS row (16-byte pad)
    constexpr int BUF = 16 * ROW;                    // floats per buffer
    constexpr int RUNS = KC / 256;                   // 1 KB runs per row (64 lanes x 16 bytes)
    constexpr int PER_WAVE = 16 * RUNS / WAVES;      // A chunk loads per wave
    typedef typename BVec<VEC>::T BT;
    __shared__ float red[WAVES][16][NW];
    __shared__ __attribute__((aligned(16))) float sa[3 * BUF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * NW;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kq = lane >> 4, lc = lane & 15;

    const rsrc_t ra = make_rsrc(p.A, clamp_extent(((int64_t)(M - 1) * lda + K) * 4));
    const float *b_strip = static_cast<const float *>(p.B) + n0;
    const uint32_t b_base = (uint32_t)(4 * kq * ldb + VEC * lc) * 4u;
    const uint32_t b_row = (uint32_t)ldb * 4u;

    f32x4 acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = f32x4{};

    // A chunk c: load j of this wave is row r = (PER_WAVE*wave + j) / RUNS,
    // run (PER_WAVE*wave + j) % RUNS, lane l's 16 bytes at k = KC*c + 256*run
    // + 4l (rows past M read row M - 1, whose products reach no stored row;
    // k past K reads as zero).
    f32x4 areg[2][PER_WAVE];
    auto load_a = [&](int set, int c) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int q = PER_WAVE * wave + j, r = q / RUNS;
            const int k = KC * c + 256 * (q % RUNS) + 4 * lane;
            areg[set][j] = __builtin_bit_cast(f32x4, load_b128(ra, k < K ? panel_off(r, M, lda, k, 4) : kOutOfRange));
        }
    };
    auto write_a = [&](int set, int c) {
        float *buf = sa + (c % 3) * BUF;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int q = PER_WAVE * wave + j;
            *reinterpret_cast<f32x4 *>(buf + (q / RUNS) * ROW + 256 * (q % RUNS) + 4 * lane) = areg[set][j];
        }
    };
    BT bv[2][UNROLL][4];
    auto issue_b = [&](int set, int t) {
        const int k0 = 16 * (t * kStride + wave);
        const rsrc_t rb = make_rsrc(b_strip + (int64_t)k0 * ldb, clamp_extent(((int64_t)(K - k0 - 1) * ldb + (N - n0)) * 4));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[set][u][j] = BVec<VEC>::load(rb, b_base + (uint32_t)(16 * u * WAVES + j) * b_row);
    };
    // Batch t: the lane's A values of block wave + u*WAVES of the chunk (row
    // lc, k = 4*kq .. 4*kq+3 of the block) against B, as in f32_skinny_kernel.
    auto consume = [&](int set, int t) {
        const float *buf = sa + (t % 3) * BUF + lc * ROW + 4 * kq;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const f32x4 av = *reinterpret_cast<const f32x4 *>(buf + 16 * (wave + u * WAVES));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int c = 0; c < VEC; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], comp<VEC>(bv[set][u][j], c), acc[c], 0, 0, 0);
        }
    };

    const int nb = (K + 15) >> 4;
    const int nbat = (nb + kStride - 1) / kStride;
    load_a(0, 0);
    load_a(1, 1);
    issue_b(0, 0);
    write_a(0, 0);
    for (int t = 0; t < nbat; t += 2) {
        issue_b(1, t + 1);               // past the end: reads zeros
        load_a(0, t + 2);
        write_a(1, t + 1);
        __syncthreads();
        consume(0, t);
        issue_b(0, t + 2);
        load_a(1, t + 3);
        write_a(0, t + 2);
        __syncthreads();
        consume(1, t + 1);
    }

    // Register r of lane (kq, lc) is row 4*kq + r, column lc of its 16 x 16 block.
#pragma unroll
    for (int c = 0; c < VEC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * kq + r][VEC * lc + c] = acc[c][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    for (int idx = tid; idx < 16 * NW; idx += 64 * WAVES) {
        const int i = idx / NW, j = idx % NW;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][i][j];
        const int col = n0 + j;
        if (i < M && col < N) {
            float v = alpha * s;
            if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
            store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
        }
    }
}

// Split-K variant for a caller-provided workspace.  Workgroup (strip, split)
// covers 64*CG columns (each lane loads 16 bytes of a k row; CG column groups
// of 64 give 256*CG contiguous bytes per row) over one of `splits` equal
// ranges of K, so B rows are read in long runs and each workgroup reads only
// its own K range of A.  The waves' partial tiles are summed in LDS and the
// workgroup stores its M x 64*CG partial to the workspace; a second kernel
// (splitk_reduce_kernel) adds the `splits` partials in split order -- the
// same order every time, so results are deterministic -- and applies alpha
// and beta.  The kernel boundary orders the two, so no device-scope fence or
// counter is needed (a fence per workgroup costs more than the reduction).
// With splits == 1 the workgroup applies the epilogue itself.
template <int CG, int VA, int WAVES, int UNROLL>
__global__ void __launch_bounds__(64 * WAVES)
f32_skinny_splitk_kernel(GemmParams p, float *partials, int splits, int kchunk) {
    constexpr int NW = 64 * CG;
    __shared__ float red[WAVES][16][NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int strip = blockIdx.x, split = blockIdx.y;
    const int n0 = strip * NW;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kbeg = split * kchunk;
    const int kend = min(K, kbeg + kchunk);
    const int kq = lane >> 4, lc = lane & 15;

    // Extents end at this split's last row, so prefetch past kend reads
    // zeros; rows of A at or past M read row M - 1.  B's resource is rebased
    // at each batch's first k row (as in the single-pass kernel).
    const rsrc_t ra = VA == 0 ? make_rsrc(static_cast<const float *>(p.A) + (int64_t)kbeg * lda,
                                          clamp_extent(((int64_t)(kend - kbeg - 1) * lda + M) * 4))
                              : make_rsrc(static_cast<const float *>(p.A) + kbeg,
                                          clamp_extent(((int64_t)(M - 1) * lda + (kend - kbeg)) * 4));
    const float *b_split = static_cast<const float *>(p.B) + (int64_t)kbeg * ldb + n0;
    const uint32_t a_base = panel_off(lc, M, lda, 4 * kq, 4);
    const uint32_t b_base = (uint32_t)(4 * kq * ldb + 4 * lc) * 4u;
    const uint32_t b_row = (uint32_t)ldb * 4u;
    const int kspan = kend - kbeg;

    f32x4 acc[CG][4];
#pragma unroll
    for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[g][c] = f32x4{};

    f32x4 av[2][UNROLL];
    f32x4 bv[2][UNROLL][4][CG];
    auto issue = [&](int set, int blk0) {
        const int k0 = 16 * blk0;
        const rsrc_t rb =
            make_rsrc(b_split + (int64_t)k0 * ldb, clamp_extent(((int64_t)(kspan - k0 - 1) * ldb + (N - n0)) * 4));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int b = blk0 + u * WAVES;
            av[set][u] = load_a_quad<VA>(ra, a_base, b, kq, lc, kspan, M, lda);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < CG; ++g)
                    bv[set][u][j][g] =
                        BVec<4>::load(rb, b_base + (uint32_t)(16 * u * WAVES + j) * b_row + 256u * g);
        }
    };
    auto consume = [&](int set) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < CG; ++g)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[g][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[set][u][j], bv[set][u][j][g][c],
                                                                         acc[g][c], 0, 0, 0);
    };

    const int nb = (kspan + 15) >> 4;
    constexpr int kStride = WAVES * UNROLL;
    issue(0, wave);
    for (int blk0 = wave; blk0 < nb; blk0 += 2 * kStride) {
        issue(1, blk0 + kStride);
        consume(0);
        issue(0, blk0 + 2 * kStride);
        consume(1);
    }

    // Register r of lane (kq, lc) in column group g, instruction c is row
    // 4*kq + r, strip column 64*g + 4*lc + c.
#pragma unroll
    for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * kq + r][64 * g + 4 * lc + c] = acc[g][c][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    if (splits == 1) {
        for (int idx = tid; idx < 16 * NW; idx += 64 * WAVES) {
            const int i = idx / NW, j = idx % NW;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s += red[w][i][j];
            const int col = n0 + j;
            if (i < M && col < N) {
                float v = alpha * s;
                if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
                store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
            }
        }
        return;
    }

    // Partial of this split -> workspace [split][M][N].
    float *mine = partials + (int64_t)split * M * N;
    for (int idx = tid; idx < 16 * NW; idx += 64 * WAVES) {
        const int i = idx / NW, j = idx % NW;
        if (i >= M || n0 + j >= N) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][i][j];
        mine[(int64_t)i * N + n0 + j] = s;
    }
}

// C = alpha * (sum over splits, in split order) + beta * C, one thread per
// output (consecutive threads along a row of C).  Every slice is loaded
// before any is added, so the loads' latencies overlap (added as they
// arrive, each load waited for the previous sum: 4.2 us for four slices of
// 16 x 8192); the sum runs in split order either way.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(GemmParams p, const float *partials, int splits) {
    const int64_t total = (int64_t)p.M * p.N;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    float part[kMaxReduceSplits];
#pragma unroll
    for (int t = 0; t < kMaxReduceSplits; ++t) {
        const float *slice = partials + (int64_t)t * total;     // uniform across the workgroup
        part[t] = t < splits ? slice[idx] : 0.0f;
    }
    float s = part[0];
#pragma unroll
    for (int t = 1; t < kMaxReduceSplits; ++t)
        if (t < splits) s += part[t];
    const int64_t i = idx / p.N, j = idx - i * p.N;
    float v = p.alpha * s;
    if (p.beta != 0.0f) v = fmaf(p.beta, p.C[i * p.ldc + j], v);
    store_out_any(p, i, j, epilogue_value(v, j, p.bias, p.act));
}

hipError_t launch_reduce(const GemmParams &p, const float *partials, int splits, hipStream_t stream) {
    if (splits < 1 || splits > kMaxReduceSplits) return hipErrorInvalidValue;
    GemmParams args = p;
    const int64_t blocks = ((int64_t)p.M * p.N + 255) / 256;
    void *argv[] = {&args, (void *)&partials, &splits};
    return hipLaunchKernel(reinterpret_cast<const void *>(&splitk_reduce_kernel), dim3((unsigned)blocks),
                           dim3(256), argv, 0, stream);
}

template <int VEC, int VA, int WAVES, int UNROLL>
hipError_t launch_f32_skinny(const GemmParams &p, hipStream_t stream) {
    const int strips = (p.N + 16 * VEC - 1) / (16 * VEC);
    GemmParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&f32_skinny_kernel<VEC, VA, WAVES, UNROLL>),
                           dim3((unsigned)strips), dim3(64 * WAVES), argv, 0, stream);
}

template <int VEC, int WAVES, int UNROLL>
hipError_t launch_f32_skinny_lds(const GemmParams &p, hipStream_t stream) {
    const int strips = (p.N + 16 * VEC - 1) / (16 * VEC);
    GemmParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&f32_skinny_lds_kernel<VEC, WAVES, UNROLL>),
                           dim3((unsigned)strips), dim3(64 * WAVES), argv, 0, stream);
}

template <int CG, int VA, int WAVES, int UNROLL>
hipError_t launch_f32_skinny_splitk(const GemmParams &p, void *workspace, hipStream_t stream) {
    const int strips = (p.N + 64 * CG - 1) / (64 * CG);
    int splits = skinny_splits(strips, p.K);
    int kchunk = ((p.K + splits - 1) / splits + 15) / 16 * 16;
    float *partials = static_cast<float *>(workspace);
    GemmParams args = p;
    void *argv[] = {&args, &partials, &splits, &kchunk};
    hipError_t err =
        hipLaunchKernel(reinterpret_cast<const void *>(&f32_skinny_splitk_kernel<CG, VA, WAVES, UNROLL>),
                        dim3((unsigned)strips, (unsigned)splits), dim3(64 * WAVES), argv, 0, stream);
    if (err != hipSuccess || splits == 1) return err;
    return launch_reduce(p, partials, splits, stream);
}

__global__ void __launch_bounds__(256)
scale_c_kernel(GemmParams p) {
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t i = idx / p.N, j = idx - i * p.N;
        const float v = p.beta == 0.0f ? 0.0f : p.beta * p.C[i * p.ldc + j];
        store_out_any(p, i, j, epilogue_value(v, j, p.bias, p.act));
    }
}

#define F32_SKINNY(VEC, VA, WAVES, UNROLL)                                                     \
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY, 16, 16 * VEC, 16 * WAVES * UNROLL, 64 * WAVES, VA, VEC,  \
     "f32_skinny_mfma16_n" #VEC "_a" #VA "_w" #WAVES "_u" #UNROLL,                              \
     &launch_f32_skinny<VEC, VA, WAVES, UNROLL>, 0, nullptr, kLayoutNN, false, kOutAll}
#define SKINNY_LIST(X)                                                                          \
    X(2, 4, 8, 4) X(2, 4, 16, 2) X(4, 4, 16, 2) X(4, 4, 8, 4) X(1, 4, 16, 4)                      \
    X(2, 1, 8, 4) X(4, 1, 16, 2) X(1, 1, 16, 2)

template __global__ void f32_skinny_splitk_kernel<2, 4, 8, 1>(GemmParams, float *, int, int);
template __global__ void f32_skinny_splitk_kernel<2, 1, 8, 1>(GemmParams, float *, int, int);
template __global__ void f32_skinny_splitk_kernel<2, 0, 8, 1>(GemmParams, float *, int, int);
template __global__ void f32_skinny_kernel<2, 0, 8, 4>(GemmParams);
template __global__ void f32_skinny_lds_kernel<2, 8, 4>(GemmParams);

// Explicit instantiations: the device pass never sees the host-only table.
#define SKINNY_INSTANTIATE(VEC, VA, WAVES, UNROLL) \
    template __global__ void f32_skinny_kernel<VEC, VA, WAVES, UNROLL>(GemmParams);
SKINNY_LIST(SKINNY_INSTANTIATE)

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// The dispatcher takes the first entry the operands allow.  2-wide loads come
// first: their 32-column strips give one workgroup per compute unit at
// N = 8192, where 4-wide strips would leave half the chip idle; 8 waves with
// 4 blocks per batch measured fastest on the 16 x 8192 x 8192 shape.
#define SKINNY_ENTRY(VEC, VA, WAVES, UNROLL) F32_SKINNY(VEC, VA, WAVES, UNROLL),
// The last entry reads A stored K x M (A transposed), with the 2-wide B
// loads and batches of the first.
const KernelDesc kF32SkinnyKernels[] = {
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY, 16, 32, 16 * 8 * 4, 512, 4, 2, "f32_skinny_mfma16_n2_alds_w8_u4",
     &launch_f32_skinny_lds<2, 8, 4>, 0, nullptr, kLayoutNN, false, kOutAll},
    SKINNY_LIST(SKINNY_ENTRY)
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY, 16, 32, 16 * 8 * 4, 512, 1, 2, "f32_skinny_mfma16_n2_at_w8_u4",
     &launch_f32_skinny<2, 0, 8, 4>, 0, nullptr, kLayoutTN, false, kOutAll},
};
const int kF32SkinnyKernelCount = sizeof(kF32SkinnyKernels) / sizeof(kF32SkinnyKernels[0]);

// Split-K skinny kernels (need the caller's workspace).  tile_n is the strip
// width; tile_k the K depth one batch of all waves covers.
const KernelDesc kF32SplitKernels[] = {
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY_SPLITK, 16, 128, 16 * 8 * 1, 512, 4, 4, "f32_skinny_splitk_n128_a4_w8_u1",
     nullptr, 0, &launch_f32_skinny_splitk<2, 4, 8, 1>, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY_SPLITK, 16, 128, 16 * 8 * 1, 512, 1, 4, "f32_skinny_splitk_n128_a1_w8_u1",
     nullptr, 0, &launch_f32_skinny_splitk<2, 1, 8, 1>, kLayoutNN, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY_SPLITK, 16, 128, 16 * 8 * 1, 512, 1, 4, "f32_skinny_splitk_n128_at_w8_u1",
     nullptr, 0, &launch_f32_skinny_splitk<2, 0, 8, 1>, kLayoutTN, false, kOutAll},
};
const int kF32SplitKernelCount = sizeof(kF32SplitKernels) / sizeof(kF32SplitKernels[0]);

hipError_t launch_splitk_reduce(const GemmParams &p, hipStream_t stream) {
    return launch_reduce(p, p.partials, k_splits(p), stream);
}

hipError_t launch_scale_c(const GemmParams &p, hipStream_t stream) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    GemmParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&scale_c_kernel), dim3((unsigned)blocks),
                           dim3(256), argv, 0, stream);
}
#endif

}  // namespace gemm
