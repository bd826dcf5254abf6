// Skinny GEMM (M <= 16) with B stored N x K: the decode-GEMV case of
// "Tiled matrix multiplication" ("Avoid when": too little reuse for tiling
// to matter, so the kernel is bound by reading B once) for weights kept
// the way a linear layer stores them, one row of K inputs per output
// column.
//
// Row n of B is then exactly what column n of the matrix instruction's B
// operand wants: each lane of v_mfma_f32_16x16x32_bf16 holds 8 consecutive
// k of one column, so a lane loads 16 contiguous bytes of its weight row
// straight into the operand, with no trip through LDS.  A (M x K, row-major)
// is read the same way: lane (row l%16, group l/16) loads 16 bytes of its
// row at the same k.  For fp32 a 16-byte load holds 4 k and feeds four
// v_mfma_f32_16x16x4_f32 instructions (instruction j takes element j of
// both operands' chunks).  Any pairing of k between lanes works as long as
// A and B use the same one.
//
//   * A k block is one 128-byte line of every row: lane group g reads bytes
//     32g .. 32g+31 as two 16-byte chunks, so a wave's two loads of a block
//     use whole lines (16-byte pieces of half lines spread over two waves
//     measured slower).
//   * A workgroup owns 32 columns of C (two 16-column groups).  Its 8 waves
//     take the k blocks round-robin, each keeping UNROLL blocks of loads in
//     flight while it consumes the previous batch; the A fragment of a block
//     serves both column groups.
//   * Workgroups are dealt to the 8 XCDs round-robin, so the 32 strips an
//     XCD runs at once are s, s+8, s+16, ...; they start at k blocks spread
//     evenly over K and wrap around.  When they all start at the same k, all
//     their rows (a power-of-two stride apart) press on the same few L2
//     channels and the kernel streams at about 3.6 TB/s instead of 4.6.
//   * The waves' 16 x 32 partial tiles are summed through LDS in wave order
//     (deterministic; no atomics), then alpha, beta and the epilogue apply.
//   * With a workspace and too few strips to cover the compute units, K is
//     also split across workgroups (grid.y); each split stores its partial
//     and the shared reduce kernel adds them in split order.
//
// For fp8 (OCP E4M3) a lane's two 16-byte chunks of a block are the 32
// consecutive k that v_mfma_f32_16x16x128_f8f6f4 wants from it, so one
// instruction takes the whole block.  That unit, like the 32x32x64 one of
// the fp8 ring kernel, sums each run of 8 consecutive k after truncating
// products below 2^-13 of the run's largest (checked with in-bounds
// probes: operand layout, random and adversarial runs, exact integers), so
// the same accuracy bound holds.  (The 32x32x64 instruction gives each
// weight row two lanes instead of four, so each load touches 32 rows; it
// streamed at 2.4 TB/s against 4.2.)
//
// With A stored K x M (AT: both operands transposed), a lane's chunk of A (the
// 16 bytes' worth of consecutive k of its row) is gathered element by
// element from the column of the stored matrix: A is at most 16 x K and
// stays in the L2s, and B still streams the same way.  Its columns at or
// past M only reach rows of C that are never written.
//
// Rows of A at or past M and rows of B at or past N lie beyond their buffer
// extents and read as zero; k blocks at or past the end of the split get an
// offset that is always out of range.  The dispatcher requires 16-byte
// aligned rows whose lengths and leading dimensions are whole 16-byte
// chunks, so a chunk is either wholly inside K or wholly past it.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

constexpr int kNtCols = 32;      // columns of C per workgroup
constexpr int kNtBlock = 128;    // bytes of every row per k block
constexpr int kNtXcds = 8;       // workgroup i runs on XCD i % 8

template <int DT> struct NtType;
// mma(a0, a1, w0, w1, acc): the lane's two 16-byte chunks of a block of A
// and of one weight row, into acc.
template <> struct NtType<GEMM_DTYPE_F32> {
    static constexpr int esz = 4;
    // Each chunk holds 4 k: four 16x16x4 instructions per chunk.
    static __device__ __forceinline__ f32x4 mma(u32x4 a0, u32x4 a1, u32x4 w0, u32x4 w1, f32x4 acc) {
        const f32x4 af[2] = {__builtin_bit_cast(f32x4, a0), __builtin_bit_cast(f32x4, a1)};
        const f32x4 wf[2] = {__builtin_bit_cast(f32x4, w0), __builtin_bit_cast(f32x4, w1)};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[h][j], wf[h][j], acc, 0, 0, 0);
        return acc;
    }
};
template <> struct NtType<GEMM_DTYPE_BF16F32> {
    static constexpr int esz = 2;
    // Each chunk = 8 consecutive k: one 16x16x32 instruction per chunk.
    static __device__ __forceinline__ f32x4 mma(u32x4 a0, u32x4 a1, u32x4 w0, u32x4 w1, f32x4 acc) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, w0),
                                                      acc, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                       __builtin_bit_cast(bf16x8, w1), acc, 0, 0, 0);
    }
};
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <> struct NtType<GEMM_DTYPE_FP8F32> {
    static constexpr int esz = 1;
    // Both chunks = 32 consecutive k: one 16x16x128 instruction (scales of
    // 2^0, so it is the unscaled operation).
    static __device__ __forceinline__ f32x4 mma(u32x4 a0, u32x4 a1, u32x4 w0, u32x4 w1, f32x4 acc) {
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const i32x8 w = {(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, w, acc, 0, 0, 0, 0, 0, 0);
    }
};

// AT: the lane's 16 bytes of A holding k = kk .. kk + 16/esz - 1 of column
// col, gathered from A stored K x M (element k at (k * lda + col) * esz of
// the resource); an offset outside the extent reads zero.
template <int DT>
__device__ __forceinline__ u32x4 gather_at(rsrc_t r, bool in, uint32_t kk, uint32_t col, uint32_t lda) {
    u32x4 v;
    if constexpr (DT == GEMM_DTYPE_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = load_b32(r, in ? ((kk + e) * lda + col) * 4u : kOutOfRange);
    } else if constexpr (DT == GEMM_DTYPE_BF16F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, in ? ((kk + 2 * e) * lda + col) * 2u : kOutOfRange, 0, 0);
            const uint32_t hi =
                __builtin_amdgcn_raw_buffer_load_b16(r, in ? ((kk + 2 * e + 1) * lda + col) * 2u : kOutOfRange, 0, 0);
            v[e] = lo | (hi << 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, in ? (kk + 4 * e + j) * lda + col : kOutOfRange, 0, 0)
                     << (8 * j);
            v[e] = w;
        }
    }
    return v;
}

template <int DT, int WAVES, int UNROLL, bool AT = false>
__global__ void __launch_bounds__(64 * WAVES)
skinny_nt_kernel(GemmParams p, float *partials, int splits, int kchunk) {
    typedef NtType<DT> E;
    constexpr int esz = E::esz;
    constexpr int kb_elems = kNtBlock / esz;   // k per block
    constexpr int chunk = 16 / esz;            // k per lane load
    __shared__ float red[WAVES][16][kNtCols];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int strip = blockIdx.x, split = blockIdx.y;
    const int n0 = strip * kNtCols;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kbeg = split * kchunk;
    const int kend = min(K, kbeg + kchunk);
    const int kspan = kend - kbeg;
    const int lc = lane & 15, g = lane >> 4;
    const int rows_here = min(kNtCols, N - n0);

    const char *A = static_cast<const char *>(p.A) + (AT ? (int64_t)kbeg * lda : (int64_t)kbeg) * esz;
    const char *W = static_cast<const char *>(p.B) + ((int64_t)n0 * ldb + kbeg) * esz;
    const rsrc_t ra = make_rsrc(A, clamp_extent((AT ? (int64_t)(kspan - 1) * lda + M : (int64_t)(M - 1) * lda + kspan) * esz));
    const rsrc_t rw = make_rsrc(W, clamp_extent(((int64_t)(rows_here - 1) * ldb + kspan) * esz));
    const uint32_t a_base = (uint32_t)(lc * lda + 2 * g * chunk) * esz;
    const uint32_t w_base0 = (uint32_t)(lc * ldb + 2 * g * chunk) * esz;
    const uint32_t w_base1 = (uint32_t)((16 + lc) * ldb + 2 * g * chunk) * esz;
    const int nb = (kspan + kb_elems - 1) / kb_elems;
    const int rot = (int)((int64_t)(strip / kNtXcds) * nb / (256 / kNtXcds) % max(nb, 1));

    f32x4 acc0 = f32x4{}, acc1 = f32x4{};
    u32x4 av[2][UNROLL][2], wv0[2][UNROLL][2], wv1[2][UNROLL][2];
    auto issue = [&](int set, int blk0) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            int b = blk0 + u * WAVES;          // blocks past nb read zeros
            const bool live = b < nb;
            b = b + rot < nb ? b + rot : b + rot - nb;
            const uint32_t koff = (uint32_t)b * kNtBlock;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool in = live && b * kb_elems + (2 * g + h) * chunk < kspan;
                if constexpr (AT)
                    av[set][u][h] = gather_at<DT>(ra, in, (uint32_t)(b * kb_elems + (2 * g + h) * chunk), (uint32_t)lc,
                                                  (uint32_t)lda);
                else
                    av[set][u][h] = load_b128(ra, in ? a_base + koff + 16u * h : kOutOfRange);
                wv0[set][u][h] = load_b128_nt(rw, in ? w_base0 + koff + 16u * h : kOutOfRange);
                wv1[set][u][h] = load_b128_nt(rw, in ? w_base1 + koff + 16u * h : kOutOfRange);
            }
        }
    };
    auto consume = [&](int set) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            acc0 = E::mma(av[set][u][0], av[set][u][1], wv0[set][u][0], wv0[set][u][1], acc0);
            acc1 = E::mma(av[set][u][0], av[set][u][1], wv1[set][u][0], wv1[set][u][1], acc1);
        }
    };

    // The scheduling barriers keep each batch's loads ahead of the previous
    // batch's instructions, so the wait before a batch covers only that
    // batch and the other set's loads stay in flight.
    constexpr int kStride = WAVES * UNROLL;
    issue(0, wave);
    for (int blk0 = wave; blk0 < nb; blk0 += 2 * kStride) {
        issue(1, blk0 + kStride);        // past the end: reads zeros
        __builtin_amdgcn_sched_barrier(0);
        consume(0);
        __builtin_amdgcn_sched_barrier(0);
        issue(0, blk0 + 2 * kStride);
        __builtin_amdgcn_sched_barrier(0);
        consume(1);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Register r of lane (g, lc) is row 4g + r, column lc of its 16-column group.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[wave][4 * g + r][lc] = acc0[r];
        red[wave][4 * g + r][16 + lc] = acc1[r];
    }
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    float *mine = splits > 1 ? partials + (int64_t)split * M * N : nullptr;
    for (int idx = tid; idx < 16 * kNtCols; idx += 64 * WAVES) {
        const int i = idx / kNtCols, j = idx % kNtCols;
        const int col = n0 + j;
        if (i >= M || col >= N) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][i][j];
        if (mine != nullptr) {
            mine[(int64_t)i * N + col] = s;
        } else {
            float v = alpha * s;
            if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
            store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
        }
    }
}

// K slices for a call: one unless a workspace lets the strips be split to
// cover the compute units; each slice is a whole number of k blocks.
template <int DT>
void nt_split(const GemmParams &p, bool with_ws, int *splits, int *kchunk) {
    constexpr int kb_elems = kNtBlock / NtType<DT>::esz;
    const int strips = (p.N + kNtCols - 1) / kNtCols;
    const int want = with_ws ? skinny_splits(strips, p.K) : 1;
    *kchunk = ((p.K + want - 1) / want + kb_elems - 1) / kb_elems * kb_elems;
    *splits = (p.K + *kchunk - 1) / *kchunk;
}

template <int DT, int WAVES, int UNROLL, bool AT = false>
hipError_t launch_nt(const GemmParams &p, void *workspace, bool with_ws, hipStream_t stream) {
    const int strips = (p.N + kNtCols - 1) / kNtCols;
    int splits, kchunk;
    nt_split<DT>(p, with_ws, &splits, &kchunk);
    float *partials = static_cast<float *>(workspace);
    GemmParams args = p;
    void *argv[] = {&args, &partials, &splits, &kchunk};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&skinny_nt_kernel<DT, WAVES, UNROLL, AT>),
                                     dim3((unsigned)strips, (unsigned)splits), dim3(64 * WAVES), argv, 0, stream);
    if (err != hipSuccess || splits == 1) return err;
    GemmParams red = p;
    red.partials = partials;
    red.kchunk = kchunk;                // k_splits(red) == splits for the shared reduce
    return launch_splitk_reduce(red, stream);
}

template <int DT, int WAVES, int UNROLL, bool AT = false>
hipError_t launch_nt_plain(const GemmParams &p, hipStream_t stream) {
    return launch_nt<DT, WAVES, UNROLL, AT>(p, nullptr, false, stream);
}
template <int DT, int WAVES, int UNROLL, bool AT = false>
hipError_t launch_nt_ws(const GemmParams &p, void *workspace, hipStream_t stream) {
    return launch_nt<DT, WAVES, UNROLL, AT>(p, workspace, true, stream);
}

template __global__ void skinny_nt_kernel<GEMM_DTYPE_F32, 8, 2>(GemmParams, float *, int, int);
template __global__ void skinny_nt_kernel<GEMM_DTYPE_BF16F32, 8, 2>(GemmParams, float *, int, int);
template __global__ void skinny_nt_kernel<GEMM_DTYPE_FP8F32, 8, 2>(GemmParams, float *, int, int);
template __global__ void skinny_nt_kernel<GEMM_DTYPE_F32, 8, 2, true>(GemmParams, float *, int, int);
template __global__ void skinny_nt_kernel<GEMM_DTYPE_BF16F32, 8, 2, true>(GemmParams, float *, int, int);
template __global__ void skinny_nt_kernel<GEMM_DTYPE_FP8F32, 8, 2, true>(GemmParams, float *, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// tile_n is the strip width; tile_k the k depth one batch of all waves
// covers; vec_a = vec_b = the elements of one 16-byte load (both operands'
// rows must be whole 16-byte chunks).  The plain entries run without a
// workspace (one slice); the split entries need one when they split.
const KernelDesc kSkinnyNtKernels[] = {
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY, 16, kNtCols, 32 * 8 * 2, 512, 4, 4, "f32_skinny_nt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_F32, 8, 2>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY, 16, kNtCols, 64 * 8 * 2, 512, 8, 8, "bf16_skinny_nt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_BF16F32, 8, 2>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 32 * 8 * 2, 512, 4, 4, "f32_skinny_nt_splitk_n32_w8_u2",
     nullptr, 0, &launch_nt_ws<GEMM_DTYPE_F32, 8, 2>, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 64 * 8 * 2, 512, 8, 8,
     "bf16_skinny_nt_splitk_n32_w8_u2", nullptr, 0, &launch_nt_ws<GEMM_DTYPE_BF16F32, 8, 2>, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY, 16, kNtCols, 128 * 8 * 2, 512, 16, 16, "fp8_skinny_nt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_FP8F32, 8, 2>, 0, nullptr, kLayoutNT, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 128 * 8 * 2, 512, 16, 16,
     "fp8_skinny_nt_splitk_n32_w8_u2", nullptr, 0, &launch_nt_ws<GEMM_DTYPE_FP8F32, 8, 2>, kLayoutNT, false, kOutAll},
    // A stored K x M as well (both operands transposed): A gathered element
    // by element, any M <= 16 and lda.
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY, 16, kNtCols, 32 * 8 * 2, 512, 1, 4, "f32_skinny_tt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_F32, 8, 2, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY, 16, kNtCols, 64 * 8 * 2, 512, 1, 8, "bf16_skinny_tt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_BF16F32, 8, 2, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    {GEMM_DTYPE_F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 32 * 8 * 2, 512, 1, 4, "f32_skinny_tt_splitk_n32_w8_u2",
     nullptr, 0, &launch_nt_ws<GEMM_DTYPE_F32, 8, 2, true>, kLayoutTT, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 64 * 8 * 2, 512, 1, 8,
     "bf16_skinny_tt_splitk_n32_w8_u2", nullptr, 0, &launch_nt_ws<GEMM_DTYPE_BF16F32, 8, 2, true>, kLayoutTT, false,
     kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY, 16, kNtCols, 128 * 8 * 2, 512, 1, 16, "fp8_skinny_tt_n32_w8_u2",
     &launch_nt_plain<GEMM_DTYPE_FP8F32, 8, 2, true>, 0, nullptr, kLayoutTT, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY_SPLITK, 16, kNtCols, 128 * 8 * 2, 512, 1, 16,
     "fp8_skinny_tt_splitk_n32_w8_u2", nullptr, 0, &launch_nt_ws<GEMM_DTYPE_FP8F32, 8, 2, true>, kLayoutTT, false,
     kOutAll},
};
const int kSkinnyNtKernelCount = sizeof(kSkinnyNtKernels) / sizeof(kSkinnyNtKernels[0]);
#endif

}  // namespace gemm
