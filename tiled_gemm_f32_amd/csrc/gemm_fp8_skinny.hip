// fp8-operand GEMM for skinny problems (M <= 16) with the weights B stored
// K x N: the decode-GEMV case that "Tiled matrix multiplication" ("Avoid
// when") identifies as bandwidth-bound, for OCP E4M3 weights kept row-major
// along N.
//
// Like the bf16 kernel of this shape (gemm_bf16_skinny.hip), the job is to
// stream B from HBM once, and the structure is that kernel's:
//
//   * Workgroup (strip, split) owns 128 columns of C over one k range; the
//     range is cut into 64-deep blocks dealt round-robin to the 4 waves, and
//     each wave sums its blocks into its own accumulators.
//   * Each wave streams its blocks into a private ring of 4 LDS slots with
//     direct-to-LDS buffer loads, so it waits only for its own loads
//     (s_waitcnt, no barrier).  A block of B is 64 k rows of 128 bytes, one
//     whole 128-byte line of every row (8 KB); A's 16 x 64-byte block (1 KB)
//     follows it in the slot.
//   * v_mfma_f32_32x32x64_f8f6f4 wants from each lane 32 consecutive k of one
//     column.  The block is laid out like a K x N slice of the 128 x 128 fp8
//     ring (16-byte chunk c of row k at chunk c ^ (k % 8)) and gathered with
//     the same byte-transposing reads, ds_read_b64_tr_b8: four per lane and
//     32-column group, 8 consecutive k each, in the same byte order as A's
//     k-contiguous 32 bytes.  The unit sums each run of 8 consecutive k as in
//     the other fp8 kernels, so their accuracy bound holds.
//   * The instruction is 32 rows tall and A has at most 16 rows: its rows
//     16 .. 31 repeat rows 0 .. 15 and their results are dropped.  Matrix
//     work does not bound this kernel; the 16-row instruction (16x16x128)
//     would need 128-deep blocks of 16 KB and a ring too large for 4 waves.
//   * With A stored K x M (AT), any M <= 16 and lda, A's 64 x 16 block is
//     loaded a byte a lane.  Such a direct-to-LDS load puts lane i's byte in
//     the low byte of dword i, the rest zero (probed), so the block takes 16
//     loads and 4 KB of dwords and the ring 3 slots of 12 KB per wave.  Load
//     j reads column j, lane l k row 4 ((l/4) ^ j) + l%4: column m's 64 k
//     then sit in 16-byte granules XOR-rotated by m, a lane's 32 k (column
//     l32 % 16) are 8 granule reads free of bank conflicts, and their low
//     bytes are packed into the fragment in k order.
//   * The waves' 16 x 128 tiles are summed through LDS in wave order; the
//     workgroup writes its partial to the caller's workspace, which the
//     shared split-order reduce kernel turns into C (alpha, beta, fused
//     epilogue).  With one split the workgroup finishes C itself.  All
//     deterministic.
#include "gemm_device.hpp"
#include "gemm_kernels.hpp"
#include "gemm.h"

namespace gemm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kKnNW = 128;                    // columns per strip (bytes of every k row)
constexpr int kKnKB = 64;                     // k per block
constexpr int kKnB = kKnKB * kKnNW;           // bytes of B per block (8 KB)
constexpr int kKnSlot = kKnB + 16 * kKnKB;    // B, then A's 16 x 64 block (1 KB)

template <int WAVES, int NSLOT, bool AT = false>
__global__ void __launch_bounds__(64 * WAVES)
fp8_skinny_kn_kernel(GemmParams p, float *partials, int splits, int kchunk) {
    static_assert(NSLOT == (AT ? 3 : 4), "four slots, three when A is loaded a byte a lane");
    constexpr int kSlot = AT ? kKnB + 4096 : kKnSlot;
    constexpr int kLoads = AT ? 24 : 9;          // loads per block: 8 of B, then A's
    // One array per slot, as in the bf16 kernel: distinct objects let the
    // compiler see that a read of one slot does not depend on loads still
    // landing in another.
    __shared__ __attribute__((aligned(1024))) char sl0[WAVES][kSlot], sl1[WAVES][kSlot], sl2[WAVES][kSlot],
        sl3[NSLOT > 3 ? WAVES : 1][NSLOT > 3 ? kSlot : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto slot_base = [&](int slot) -> char * {
        return slot == 0 ? sl0[wave] : slot == 1 ? sl1[wave] : (NSLOT == 3 || slot == 2) ? sl2[wave] : sl3[wave];
    };
    const int strip = blockIdx.x, split = blockIdx.y;
    const int n0 = strip * kKnNW;
    const int M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int kbeg = split * kchunk;
    const int kspan = min(K, kbeg + kchunk) - kbeg;
    const int h = lane >> 5, l32 = lane & 31, s16 = lane & 15;

    // B is addressed through resources rebased at each block's first k row,
    // with extents ending at the range's last k row (rows past the range read
    // as zero; offsets span one 64-row block whatever the operand's size).  A
    // has one resource ending after its last valid element (the host keeps it
    // below 2^31 bytes); its rows at or past M read row M - 1, which only
    // reaches rows of C that are never written, and its chunks past the range
    // get an offset outside every extent, as a zero of B times an infinity
    // there would not vanish.  Columns past N hold whatever follows in memory
    // (or zero past the extent) and only reach columns of C that are never
    // written.
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    const rsrc_t ra = make_rsrc(A + kbeg, clamp_extent((int64_t)(M - 1) * lda + kspan));
    const uint8_t *b_range = B + (int64_t)kbeg * ldb + n0;
    const uint8_t *a_range = A + (int64_t)kbeg * lda;     // A stored K x M

    // Load i (0..7) of a block: k rows 8i .. 8i+7; lane -> row 8i + lane/8,
    // physical chunk lane%8 holding logical chunk (lane%8) ^ (row%8).  It
    // lands at slot + 1024 i + 16 lane.
    uint32_t b_goff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kr = 8 * i + (lane >> 3);
        b_goff[i] = (uint32_t)kr * (uint32_t)ldb + 16u * (uint32_t)((lane & 7) ^ (kr & 7));
    }
    // A's load: lane -> row lane/4, 16-byte chunk lane%4 (k = 16 (lane%4) ..,
    // the first of which is a_kc), at slot + kKnB + 16 lane (row-major, 64
    // bytes a row).
    const uint32_t a_goff = panel_off(lane >> 2, M, lda, 16 * (lane & 3), 1);
    const int a_kc = 16 * (lane & 3);
    // A fragment: lane (h, l32) holds row l32 % 16, bytes 32h .. 32h+31.
    const uint32_t a_read = (uint32_t)(kKnB + (l32 & 15) * kKnKB + 32 * h);
    // AT: load j's offset of lane l (k row 4 ((l/4) ^ j) + l%4, column j),
    // and the base of the lane's granule reads (column l32 % 16).
    uint32_t at_goff[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        at_goff[j] = (uint32_t)(4 * ((lane >> 2) ^ j) + (lane & 3)) * (uint32_t)lda + (uint32_t)j;
    const int at_m = l32 & 15;
    const uint32_t at_read = (uint32_t)(kKnB + 256 * at_m);
    // B fragment of column group g (32 columns), part q (8 k): lane s16 of
    // each 16-lane group points at k row 32h + 8q + e(s16) and at half
    // 8 (s16 % 2) of the chunk holding its group's 16 columns, so that lane
    // l32 receives k 32h + 8q .. +7 of column 32g + l32.
    const int e_src = ((s16 >> 1) & 3) + 4 * (s16 >> 3);
    uint32_t tr_off[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kr = 32 * h + 8 * q + e_src;
            const int c = 2 * g + (l32 >> 4);
            tr_off[g][q] = (uint32_t)(kr * kKnNW + 16 * (c ^ (kr & 7)) + 8 * (s16 & 1));
        }

    const int nb = (kspan + kKnKB - 1) / kKnKB;
    f32x16 acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = f32x16{};

    // Block t of this wave is block wave + t*WAVES of the range; it goes to
    // slot t % NSLOT.  kLoads loads per block: 8 of B, then A's.
    auto issue = [&](int t, int slot) {
        const int k0 = (wave + t * WAVES) * kKnKB;
        const rsrc_t rb =
            make_rsrc(b_range + (int64_t)k0 * ldb, clamp_extent((int64_t)(kspan - k0 - 1) * ldb + (N - n0)));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(slot_base(slot) + 1024 * i), 16, b_goff[i], 0, 0,
                                                     0);
        if constexpr (AT) {
            const rsrc_t rat =
                make_rsrc(a_range + (int64_t)k0 * lda, clamp_extent((int64_t)(kspan - k0 - 1) * lda + M));
#pragma unroll
            for (int j = 0; j < 16; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rat, (lds_void *)(slot_base(slot) + kKnB + 256 * j), 1,
                                                         at_goff[j], 0, 0, 0);
        } else {
            const uint32_t off = k0 + a_kc >= kspan ? kOutOfRange : a_goff + (uint32_t)k0;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(slot_base(slot) + kKnB), 16, off, 0, 0, 0);
        }
    };
    auto consume = [&](int slot) {
        const char *base = slot_base(slot);
        i32x8 fa;
        if constexpr (AT) {
            // Granule i of the lane's k range (k 32h + 4i ..) is physical
            // granule (8h + i) ^ m of column m's 64 dwords.
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(base + at_read + 16 * ((8 * h + i) ^ at_m));
                fa[i] = (int)(v[0] | (v[1] << 8) | (v[2] << 16) | (v[3] << 24));
            }
        } else {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(base + a_read);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(base + a_read + 16);
            fa = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            i32x8 fb;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(base + tr_off[g][q]));
                fb[2 * q] = v[0];
                fb[2 * q + 1] = v[1];
            }
            acc[g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[g], 0, 0, 0, 0, 0, 0);
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

    // Register 4j + t of lane (h, l32) in column group g is row l32 (rows 16
    // .. 31 repeat 0 .. 15), column 32g + 8j + 4h + t.  16 x 128 fp32 per wave
    // = 8 KB: the reduction reuses the slot-0 arrays.
    static_assert(WAVES * 16 * kKnNW * 4 <= sizeof(sl0), "slot 0 holds every wave's tile");
    float(*red)[16][kKnNW] = reinterpret_cast<float(*)[16][kKnNW]>(&sl0[0][0]);
    if (l32 < 16) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) red[wave][l32][32 * g + 8 * j + 4 * h + t] = acc[g][4 * j + t];
    }
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    float *mine = splits > 1 ? partials + (int64_t)split * M * N : nullptr;
    for (int idx = tid; idx < 16 * kKnNW; idx += 64 * WAVES) {
        const int i = idx / kKnNW, j = idx % kKnNW;
        const int col = n0 + j;
        if (i >= M || col >= N) continue;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += red[w][i][j];
        if (mine != nullptr) {
            mine[(int64_t)i * N + col] = sum;          // partial of this split -> workspace [split][M][N]
        } else {
            float v = alpha * sum;
            if (beta != 0.0f) v = fmaf(beta, p.C[(int64_t)i * p.ldc + col], v);
            store_out_any(p, i, col, epilogue_value(v, col, p.bias, p.act));
        }
    }
}

// SPLIT: cut K over workgroups as skinny_splits() suggests (which needs the
// workspace); otherwise every workgroup covers the whole of K and finishes C.
// Each split is a whole number of 64-deep blocks.
template <int WAVES, int NSLOT, bool SPLIT = true, bool AT = false>
hipError_t launch_fp8_skinny_kn(const GemmParams &p, void *workspace, hipStream_t stream) {
    const int strips = (p.N + kKnNW - 1) / kKnNW;
    const int want = SPLIT ? skinny_splits(strips, p.K) : 1;
    const int kchunk = ((p.K + want - 1) / want + kKnKB - 1) / kKnKB * kKnKB;
    int splits = (p.K + kchunk - 1) / kchunk;     // never more than the workspace was sized for
    GemmParams args = p;
    float *partials = static_cast<float *>(workspace);
    int kc = kchunk;
    void *argv[] = {&args, &partials, &splits, &kc};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&fp8_skinny_kn_kernel<WAVES, NSLOT, AT>),
                                     dim3((unsigned)strips, (unsigned)splits), dim3(64 * WAVES), argv, 0, stream);
    if (err != hipSuccess || splits == 1) return err;
    GemmParams red = p;
    red.partials = partials;
    red.kchunk = kchunk;                // k_splits(red) == splits for the shared reduce
    return launch_splitk_reduce(red, stream);
}

template <int WAVES, int NSLOT, bool AT = false>
hipError_t launch_fp8_skinny_kn_whole_k(const GemmParams &p, hipStream_t stream) {
    return launch_fp8_skinny_kn<WAVES, NSLOT, false, AT>(p, nullptr, stream);
}

template __global__ void fp8_skinny_kn_kernel<4, 4, false>(GemmParams, float *, int, int);
template __global__ void fp8_skinny_kn_kernel<4, 3, true>(GemmParams, float *, int, int);

}  // namespace

#if !defined(__HIP_DEVICE_COMPILE__)
// tile_n is the strip width; tile_k the k depth of one block.  vec_a =
// vec_b = 16: 16-byte loads of both (rows whole 16-byte chunks, 16-byte
// aligned); other operands take the tiled kernels.
const KernelDesc kFp8SkinnyKernels[] = {
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY_SPLITK, 16, kKnNW, kKnKB, 256, 16, 16, "fp8_skinny_kn_n128_w4_s4",
     nullptr, 0, &launch_fp8_skinny_kn<4, 4, true, false>, kLayoutNN, false, kOutAll},
    // Without a workspace: one workgroup per strip over the whole of K.
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY, 16, kKnNW, kKnKB, 256, 16, 16, "fp8_skinny_kn_n128_w4_s4_whole_k",
     &launch_fp8_skinny_kn_whole_k<4, 4>, 0, nullptr, kLayoutNN, false, kOutAll},
    // A stored K x M (any M <= 16, lda or alignment), loaded a byte a lane.
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY_SPLITK, 16, kKnNW, kKnKB, 256, 1, 16, "fp8_skinny_kn_at1_n128_w4_s3",
     nullptr, 0, &launch_fp8_skinny_kn<4, 3, true, true>, kLayoutTN, false, kOutAll},
    {GEMM_DTYPE_FP8F32, GEMM_PATH_SKINNY, 16, kKnNW, kKnKB, 256, 1, 16, "fp8_skinny_kn_at1_n128_w4_s3_whole_k",
     &launch_fp8_skinny_kn_whole_k<4, 3, true>, 0, nullptr, kLayoutTN, false, kOutAll},
};
const int kFp8SkinnyKernelCount = sizeof(kFp8SkinnyKernels) / sizeof(kFp8SkinnyKernels[0]);
#endif

}  // namespace gemm
