// bf16-operand GEMM for skinny problems (M <= 16): the decode-GEMV case that
// "Tiled matrix multiplication" ("Avoid when") identifies as bandwidth-bound,
// with bf16 weights (B).
//
// With at most 16 rows of A, each byte of B feeds one multiply-add per row,
// so the job is to stream B from HBM once at full bandwidth.  Widening B to
// fp32 and using the fp32 matrix instruction costs one 32-cycle instruction
// per 4 columns x 4 k of B, which is about as long as those bytes take to
// arrive; the bf16 instruction v_mfma_f32_16x16x32_bf16 does 32 k at once.
// It wants each lane to hold 8 consecutive k of one column of B, while B's
// rows hold consecutive columns, so B goes through LDS:
//
//   * Workgroup (strip, split) owns 128 columns of C over one k range (the
//     split-K form of "Tiled matrix multiplication", "Variants and
//     alternatives").  The range is cut into 32-deep blocks dealt
//     round-robin to the waves; each wave sums its blocks into its own
//     16 x 128 tile.
//   * Each wave streams its blocks into a private ring of NSLOT LDS slots
//     with direct-to-LDS buffer loads (8 KB per block: 32 rows of 256
//     bytes), so it waits only for its own loads (s_waitcnt, no barrier).
//   * The transposing read ds_read_b64_tr_b16 turns 4 rows x 16 columns into
//     one column's 4 k values per lane (the B operand layout of the matrix
//     instruction); two of them give the 8.  16-byte chunks of a row are
//     XOR-swizzled by the row so that the 16 rows one read touches spread over
//     the 64 banks (each half-wave conflict-free).
//   * A's 16 x 32 block comes along in the same slot (one more 1 KB load)
//     and is read back 8 consecutive k per lane, so every load in the loop
//     goes to LDS and the wait for a slot is the wait for its own loads.
//   * The waves' tiles are summed through LDS in wave order; the workgroup
//     writes its partial to the caller's workspace, which the shared
//     split-order reduce kernel turns into C (alpha, beta, fused epilogue).
//     With one split the workgroup finishes C itself.  All deterministic.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

constexpr int kSkNW = 128;             // columns per strip
constexpr int kSkKB = 32;              // k per block
constexpr int kSkB = kSkKB * kSkNW * 2;      // bytes of B per block (8 KB)
constexpr int kSkSlot = kSkB + 16 * kSkKB * 2;   // B, then A's 16 x 32 block (1 KB)

// Swizzle of the 16-byte chunks (16 per 256-byte row): XOR by an even value,
// so the two chunks a lane group reads together stay adjacent.  Rows 8q + t
// (q = 0..3, t = 0..7) of one read get (t & 3) + 4 (q & 1) pairs apart.
__device__ __forceinline__ int sk_swz(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }

// AT: A is stored K x M (M and lda multiples of 8).  Its 32 x 16 block of a
// slot is then 32 rows of 32 bytes (lane -> k row lane/2, half lane%2) and
// the A operand comes out of the same transposing reads as B's (one
// 16-column block: lane s gets column m = s).  Columns of the stored block
// at or past M only reach rows of C that are never written.
//
// AV = 1 (with AT): A stored K x M with any M <= 16 and lda, loaded 2 bytes
// a lane.  Such a direct-to-LDS load places lane i's element in the low half
// of dword i (probed), so the block takes 8 loads and 2 KB of dwords (and the
// ring the whole 160 KB of LDS).  Load j, lane l holds k row 4j + (l/16 ^
// (j/2 % 4)), column l % 16 of the block: each load reads 16 consecutive
// columns of four rows, and the A fragment (lane (q, s): column s, k 8q ..
// 8q+7) is read back as 8 dwords whose banks differ across the four q.
template <int WAVES, int NSLOT, bool AT = false, int AV = 8>
__global__ void __launch_bounds__(64 * WAVES)
bf16_skinny_kernel(GemmParams p, float *partials, int splits, int kchunk) {
    static_assert(NSLOT == 4, "four slot arrays");
    static_assert(AV == 8 || (AT && AV == 1), "A loaded 16 bytes a lane, or 2 bytes when stored K x M");
    constexpr bool kA2 = AV == 1;
    constexpr int kSlot = kA2 ? kSkB + 2048 : kSkSlot;
    constexpr int kLoads = kA2 ? 16 : 9;       // loads per block: 8 of B, then A's
    // One array per slot: with distinct objects the compiler can tell that a
    // read of one slot does not depend on loads still landing in another, and
    // does not wait for the whole ring.
    __shared__ __attribute__((aligned(1024))) char sl0[WAVES][kSlot], sl1[WAVES][kSlot], sl2[WAVES][kSlot],
        sl3[WAVES][kSlot];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto slot_base = [&](int slot) -> char * {
        return slot == 0 ? sl0[wave] : slot == 1 ? sl1[wave] : slot == 2 ? sl2[wave] : sl3[wave];
    };
    const int strip = blockIdx.x, split = blockIdx.y;
    const int n0 = strip * kSkNW;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kbeg = split * kchunk;
    const int kspan = min(K, kbeg + kchunk) - kbeg;
    const int q = lane >> 4, s = lane & 15;

    // B (and A stored K x M) are addressed through resources rebased at each
    // block's first k row, with extents ending at the range's last k row: rows
    // past the range read as zero, and offsets span one 32-row block whatever
    // the size of the operand.  A stored M x K has one resource ending after
    // its last valid element (the host keeps it below 2^31 bytes); its rows
    // at or past M read row M - 1, which only reaches rows of C that are never
    // written, and its chunks past the range (which hold the next range's k)
    // are given an offset outside every extent, as a zero of B times an
    // infinity there would not vanish.
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    const rsrc_t ra_mk = make_rsrc(A + kbeg, clamp_extent(((int64_t)(M - 1) * lda + kspan) * 2));
    const uint16_t *b_range = B + (int64_t)kbeg * ldb + n0;
    const uint16_t *a_range = A + (int64_t)kbeg * lda;     // A stored K x M

    // Load instruction i (0..7) of a block: rows 4i .. 4i+3; lane -> row
    // 4i + lane/16, physical chunk lane%16 holding logical chunk
    // (lane%16) ^ swizzle(row).  It lands at slot + 1024 i + 16 lane.
    uint32_t b_goff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + (lane >> 4);
        const int lc = (lane & 15) ^ sk_swz(row);
        b_goff[i] = (uint32_t)(row * ldb + 8 * lc) * 2u;
    }
    // Transposing reads: lane s of group q points at row 8q + s/4 (+4 for
    // the second read), columns 16 cb + 4 (s%4) .. +3 of column block cb.
    uint32_t tr_off[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const int row = 8 * q + (s >> 2) + 4 * h;
            const int col = 16 * cb + 4 * (s & 3);
            const int chunk = (col >> 3) ^ sk_swz(row);
            tr_off[h][cb] = (uint32_t)(row * 256 + 16 * chunk + 2 * (col & 7));
        }
    // A's load: lane -> row lane/4, 16-byte chunk lane%4 (k = 8 (lane%4) ..,
    // the first of which is a_kc); with AT, lane -> k row lane/2 of the block,
    // columns 8 (lane%2) .. +7.
    const uint32_t a_goff = AT ? (uint32_t)((lane >> 1) * lda + 8 * (lane & 1)) * 2u
                               : panel_off(lane >> 2, M, lda, 8 * (lane & 3), 2);
    const int a_kc = 8 * (lane & 3);
    const uint32_t a_read = (uint32_t)(kSkB + s * 64 + 16 * q);
    // AT: lane s of group q points at k row 8q + s/4 (+4), columns 4 (s%4) .. +3.
    uint32_t at_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) at_off[h] = (uint32_t)(kSkB + (8 * q + (s >> 2) + 4 * h) * 32 + 8 * (s & 3));
    // AV = 1: load j reads k rows 4j .. 4j+3, lane l row 4j + (l/16 ^ c) with
    // c = j/2 % 4 (offset a2_goff[c] + j * a2_step).  Fragment element i
    // (k = 8q + i) then sits in dword 64 (2q + i/4) + 16 ((i%4) ^ q) + s of
    // the block.
    uint32_t a2_goff[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) a2_goff[c] = (uint32_t)((((lane >> 4) ^ c) * lda + (lane & 15)) * 2);
    const uint32_t a2_step = (uint32_t)(8 * lda);
    const uint32_t a2_read = (uint32_t)(kSkB + 512 * q + 4 * s);

    const int nb = (kspan + kSkKB - 1) / kSkKB;
    f32x4 acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4{};

    // Block t of this wave is block wave + t*WAVES of the range; it goes to
    // slot t % NSLOT.  kLoads loads per block: 8 of B, then A's.
    auto issue = [&](int t, int slot) {
        const int k0 = (wave + t * WAVES) * kSkKB;
        const rsrc_t rb = make_rsrc(b_range + (int64_t)k0 * ldb, clamp_extent(((int64_t)(kspan - k0 - 1) * ldb + (N - n0)) * 2));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(slot_base(slot) + 1024 * i), 16, b_goff[i], 0, 0,
                                                     0);
        if constexpr (kA2) {
            const rsrc_t ra = make_rsrc(a_range + (int64_t)k0 * lda, clamp_extent(((int64_t)(kspan - k0 - 1) * lda + M) * 2));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(slot_base(slot) + kSkB + 256 * j), 2,
                                                         a2_goff[(j >> 1) & 3] + (uint32_t)j * a2_step, 0, 0, 0);
        } else if constexpr (AT) {
            const rsrc_t ra = make_rsrc(a_range + (int64_t)k0 * lda, clamp_extent(((int64_t)(kspan - k0 - 1) * lda + M) * 2));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(slot_base(slot) + kSkB), 16, a_goff, 0, 0, 0);
        } else {
            const uint32_t off = k0 + a_kc >= kspan ? kOutOfRange : a_goff + (uint32_t)k0 * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_mk, (lds_void *)(slot_base(slot) + kSkB), 16, off, 0, 0, 0);
        }
    };
    auto consume = [&](int slot) {
        const char *base = slot_base(slot);
        bf16x8 afrag;
        if constexpr (kA2) {
            typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
            u16x8 e;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                e[i] = *reinterpret_cast<const uint16_t *>(base + a2_read + 256 * (i >> 2) + 64 * ((i & 3) ^ q));
            afrag = __builtin_bit_cast(bf16x8, e);
        } else if constexpr (AT) {
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + at_off[0]));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + at_off[1]));
            afrag = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            afrag = *reinterpret_cast<const bf16x8 *>(base + a_read);
        }
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_off[0][cb]));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(base + tr_off[1][cb]));
            const bf16x8 bfrag = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc[cb], 0, 0, 0);
        }
    };

    const int my_blocks = nb > wave ? (nb - wave + WAVES - 1) / WAVES : 0;
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) issue(t, t);      // past the range: zeros
    for (int t0 = 0; t0 < my_blocks; t0 += NSLOT) {
#pragma unroll
        for (int u = 0; u < NSLOT; ++u) {
            // Block t0+u has landed once at most the kLoads loads of each
            // later block are outstanding; then its slot is read and refilled.
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kLoads * (NSLOT - 1)));
            if (t0 + u < my_blocks) consume(u);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kLoads * (NSLOT - 1)));   // reads done before the refill
            issue(t0 + u + NSLOT, u);
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();

    // Register r of lane (q, s) in column block cb is row 4q + r, column 16 cb + s.
    // 16 x 128 fp32 per wave = 8 KB: the reduction reuses the slot-0 arrays.
    static_assert(WAVES * 16 * kSkNW * 4 <= sizeof(sl0), "slot 0 holds every wave's tile");
    float(*red)[16][kSkNW] = reinterpret_cast<float(*)[16][kSkNW]>(&sl0[0][0]);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * q + r][16 * cb + s] = acc[cb][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    if (splits == 1) {
        for (int idx = tid; idx < 16 * kSkNW; idx += 64 * WAVES) {
            const int i = idx / kSkNW, j = idx % kSkNW;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) sum += red[w][i][j];
            const int col = n0 + j;
            if (i < M && col < N) {
                float v = alpha * sum;
                if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
                store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
            }
        }
        return;
    }
    // Partial of this split -> workspace [split][M][N].
    float *mine = partials + (int64_t)split * M * N;
    for (int idx = tid; idx < 16 * kSkNW; idx += 64 * WAVES) {
        const int i = idx / kSkNW, j = idx % kSkNW;
        if (i >= M || n0 + j >= N) continue;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += red[w][i][j];
        mine[(int64_t)i * N + n0 + j] = sum;
    }
}

// SPLIT: cut K over workgroups as skinny_splits() suggests (which needs the
// workspace); otherwise every workgroup covers the whole of K and finishes C.
template <int WAVES, int NSLOT, bool SPLIT = true, bool AT = false, int AV = 8>
hipError_t launch_bf16_skinny(const GemmParams &p, void *workspace, hipStream_t stream) {
    const int strips = (p.N + kSkNW - 1) / kSkNW;
    const int want = SPLIT ? skinny_splits(strips, p.K) : 1;
    int kchunk = ((p.K + want - 1) / want + 15) / 16 * 16;
    int splits = (p.K + kchunk - 1) / kchunk;     // never more than the workspace was sized for
    GemmParams args = p;
    float *partials = static_cast<float *>(workspace);
    void *argv[] = {&args, &partials, &splits, &kchunk};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&bf16_skinny_kernel<WAVES, NSLOT, AT, AV>),
                                     dim3((unsigned)strips, (unsigned)splits), dim3(64 * WAVES), argv, 0, stream);
    if (err != hipSuccess || splits == 1) return err;
    GemmParams red = p;
    red.partials = partials;
    red.kchunk = kchunk;                // k_splits(red) == splits for the shared reduce
    return launch_splitk_reduce(red, stream);
}

template <int WAVES, int NSLOT, bool AT = false, int AV = 8>
hipError_t launch_bf16_skinny_whole_k(const GemmParams &p, hipStream_t stream) {
    return launch_bf16_skinny<WAVES, NSLOT, false, AT, AV>(p, nullptr, stream);
}

template __global__ void bf16_skinny_kernel<4, 4, false>(GemmParams, float *, int, int);
template __global__ void bf16_skinny_kernel<4, 4, true>(GemmParams, float *, int, int);
template __global__ void bf16_skinny_kernel<4, 4, true, 1>(GemmParams, float *, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// tile_n is the strip width; tile_k the k depth of one block.  vec_a =
// vec_b = 8: 16-byte loads of both (rows whole 16-byte chunks, 16-byte
// aligned); other operands take the tiled kernels.
const KernelDesc kBf16SplitKernels[] = {
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY_SPLITK, 16, kSkNW, kSkKB, 256, 8, 8, "bf16_skinny_lds_n128_w4_s4",
     nullptr, 0, &launch_bf16_skinny<4, 4>, kLayoutNN, false, kOutAll},
    // Without a workspace: one workgroup per strip over the whole of K.  At
    // N = 8192 that is 64 workgroups, still far ahead of the tiled kernels,
    // which compute 128 rows for 16 on as many workgroups.
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY, 16, kSkNW, kSkKB, 256, 8, 8, "bf16_skinny_lds_n128_w4_s4_whole_k",
     &launch_bf16_skinny_whole_k<4, 4>, 0, nullptr, kLayoutNN, false, kOutAll},
    // A stored K x M: its K rows (M long) must be whole 16-byte chunks too,
    // so M is 8 or 16.  Then the extent of each split's A ends on a chunk
    // boundary; a 16-byte load that straddled it would read as zero whole.
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY_SPLITK, 16, kSkNW, kSkKB, 256, 8, 8, "bf16_skinny_lds_n128_at_w4_s4",
     nullptr, 0, &launch_bf16_skinny<4, 4, true, true>, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY, 16, kSkNW, kSkKB, 256, 8, 8, "bf16_skinny_lds_n128_at_w4_s4_whole_k",
     &launch_bf16_skinny_whole_k<4, 4, true>, 0, nullptr, kLayoutTN, false, kOutAll},
    // A stored K x M otherwise (any M <= 16, lda or alignment): loaded 2
    // bytes a lane.
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY_SPLITK, 16, kSkNW, kSkKB, 256, 1, 8, "bf16_skinny_lds_n128_at1_w4_s4",
     nullptr, 0, &launch_bf16_skinny<4, 4, true, true, 1>, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_BF16F32, GEMM_PATH_SKINNY, 16, kSkNW, kSkKB, 256, 1, 8, "bf16_skinny_lds_n128_at1_w4_s4_whole_k",
     &launch_bf16_skinny_whole_k<4, 4, true, 1>, 0, nullptr, kLayoutTN, false, kOutAll},
};
const int kBf16SplitKernelCount = sizeof(kBf16SplitKernels) / sizeof(kBf16SplitKernels[0]);
#endif

}  // namespace gemm
