// The C ABI of libgemm: argument validation, kernel choice and launch.
//
// Everything up to the launch is plain host arithmetic on the arguments, so
// a bad call is rejected before any HIP call and the choice can be inspected
// on a machine without a GPU (gemm_plan_query).  The choice follows the
// pages' reasoning about tiles and waves ("A GEMM Kernel, Step by Step",
// sections "The fringe and the last wave" and "Six parameters, found by
// search"): the largest workgroup tile that still gives every compute unit
// work, the widest global loads the operands' alignment permits, and a
// separate streaming kernel for M <= 16.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "gemm.h"
#include "gemm_kernels.hpp"

namespace {

using gemm::KernelDesc;

constexpr int64_t kMaxDim = 0x7fffffff;   // sizes and leading dimensions index with 32-bit integers in the kernels
constexpr int kComputeUnits = 256;

int table_size() {
    return gemm::kF32TiledKernelCount + gemm::kBf16TiledKernelCount + gemm::kF32SkinnyKernelCount +
           gemm::kF32SplitKernelCount + gemm::kFp8TiledKernelCount + gemm::kGeneralKernelCount +
           gemm::kBf16SplitKernelCount + gemm::kSkinnyNtKernelCount + gemm::kBf16LinesKernelCount +
           gemm::kFp8LinesKernelCount + gemm::kFp8SkinnyKernelCount;
}

const KernelDesc *kernel_by_id(int32_t id) {
    if (id < 1) return nullptr;
    int i = id - 1;
    if (i < gemm::kF32TiledKernelCount) return &gemm::kF32TiledKernels[i];
    i -= gemm::kF32TiledKernelCount;
    // The line-granular bf16 kernel comes before the other bf16 kernels: the
    // automatic choice takes the first kernel of a tile size that runs a call.
    if (i < gemm::kBf16LinesKernelCount) return &gemm::kBf16LinesKernels[i];
    i -= gemm::kBf16LinesKernelCount;
    if (i < gemm::kBf16TiledKernelCount) return &gemm::kBf16TiledKernels[i];
    i -= gemm::kBf16TiledKernelCount;
    if (i < gemm::kF32SkinnyKernelCount) return &gemm::kF32SkinnyKernels[i];
    i -= gemm::kF32SkinnyKernelCount;
    if (i < gemm::kF32SplitKernelCount) return &gemm::kF32SplitKernels[i];
    i -= gemm::kF32SplitKernelCount;
    // Likewise the line-granular fp8 kernel before the fp8 rings.
    if (i < gemm::kFp8LinesKernelCount) return &gemm::kFp8LinesKernels[i];
    i -= gemm::kFp8LinesKernelCount;
    if (i < gemm::kFp8TiledKernelCount) return &gemm::kFp8TiledKernels[i];
    i -= gemm::kFp8TiledKernelCount;
    if (i < gemm::kGeneralKernelCount) return &gemm::kGeneralKernels[i];
    i -= gemm::kGeneralKernelCount;
    if (i < gemm::kBf16SplitKernelCount) return &gemm::kBf16SplitKernels[i];
    i -= gemm::kBf16SplitKernelCount;
    if (i < gemm::kSkinnyNtKernelCount) return &gemm::kSkinnyNtKernels[i];
    i -= gemm::kSkinnyNtKernelCount;
    if (i < gemm::kFp8SkinnyKernelCount) return &gemm::kFp8SkinnyKernels[i];
    return nullptr;
}

int32_t id_of(const KernelDesc *kd) {
    for (int32_t id = 1; id <= table_size(); ++id)
        if (kernel_by_id(id) == kd) return id;
    return 0;
}

bool aligned(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Call {
    int32_t dtype;
    int32_t op_a, op_b;    // gemm_op layouts
    int64_t M, N, K;
    float alpha, beta;
    const void *A, *B;
    float *C;
    int64_t lda, ldb, ldc;
    void *ws;
    int64_t ws_bytes;
    const float *bias;     // fused epilogue (null: none)
    int32_t act;           // gemm_activation
    int32_t out_type;      // gemm_output
    void *out;             // bf16 / fp8 output (out_type != GEMM_OUT_F32)
    int64_t ldo;
    float out_scale;
};

int elem_size(int32_t dtype) { return dtype == GEMM_DTYPE_F32 ? 4 : dtype == GEMM_DTYPE_BF16F32 ? 2 : 1; }

// Length of each operand's stored rows (its contiguous dimension).
int64_t row_len_a(const Call &c) { return c.op_a == GEMM_OP_N ? c.K : c.M; }
int64_t row_len_b(const Call &c) { return c.op_b == GEMM_OP_N ? c.N : c.K; }

gemm_status validate(const Call &c) {
    if (c.dtype != GEMM_DTYPE_F32 && c.dtype != GEMM_DTYPE_BF16F32 && c.dtype != GEMM_DTYPE_FP8F32)
        return GEMM_ERR_INVALID_ARG;
    if ((c.op_a != GEMM_OP_N && c.op_a != GEMM_OP_T) || (c.op_b != GEMM_OP_N && c.op_b != GEMM_OP_T))
        return GEMM_ERR_INVALID_ARG;
    if (c.M < 0 || c.N < 0 || c.K < 0) return GEMM_ERR_INVALID_ARG;
    const int64_t min_lda = row_len_a(c) > 1 ? row_len_a(c) : 1;
    const int64_t min_ldb = row_len_b(c) > 1 ? row_len_b(c) : 1;
    const int64_t min_ldc = c.N > 1 ? c.N : 1;
    if (c.lda < min_lda || c.ldb < min_ldb || c.ldc < min_ldc) return GEMM_ERR_INVALID_ARG;
    if (c.ws_bytes < 0 || (c.ws != nullptr && !aligned(c.ws, 4))) return GEMM_ERR_INVALID_ARG;
    if (c.act < GEMM_ACT_NONE || c.act > GEMM_ACT_GELU) return GEMM_ERR_INVALID_ARG;
    if (c.bias != nullptr && !aligned(c.bias, 4)) return GEMM_ERR_INVALID_ARG;
    if (c.out_type < GEMM_OUT_F32 || c.out_type > GEMM_OUT_FP8) return GEMM_ERR_INVALID_ARG;
    if (c.out_type != GEMM_OUT_F32) {
        const int64_t min_ldo = c.N > 1 ? c.N : 1;
        if (c.ldo < min_ldo || !aligned(c.out, c.out_type == GEMM_OUT_BF16 ? 2 : 1)) return GEMM_ERR_INVALID_ARG;
        if (c.out == nullptr && c.M > 0 && c.N > 0) return GEMM_ERR_INVALID_ARG;
        if (c.ldo > kMaxDim) return GEMM_ERR_UNSUPPORTED;
    }
    if (c.C != nullptr && !aligned(c.C, 4)) return GEMM_ERR_INVALID_ARG;
    const uintptr_t esz = (uintptr_t)elem_size(c.dtype);
    if (c.M > 0 && c.N > 0) {
        // C is written for fp32 output and read as C0 when beta != 0.
        if (c.C == nullptr && (c.out_type == GEMM_OUT_F32 || c.beta != 0.0f)) return GEMM_ERR_INVALID_ARG;
        if (c.K > 0 && c.alpha != 0.0f) {
            if (c.A == nullptr || c.B == nullptr || !aligned(c.A, esz) || !aligned(c.B, esz))
                return GEMM_ERR_INVALID_ARG;
        }
    }
    if (c.M > kMaxDim || c.N > kMaxDim || c.K > kMaxDim) return GEMM_ERR_UNSUPPORTED;
    if (c.lda > kMaxDim || c.ldb > kMaxDim) return GEMM_ERR_UNSUPPORTED;
    return GEMM_OK;
}

// Widest vector loads each operand allows: 16-byte aligned base, leading
// dimension and extent along the contiguous axis multiples of the width (so
// a vector is either wholly inside the valid region or wholly outside).
bool vec_ok(const void *p, int64_t ld, int64_t row_len, int esz, int v) {
    return v == 1 || (aligned(p, (uintptr_t)(esz * v)) && ld % v == 0 && row_len % v == 0);
}
int max_vec_a(const Call &c) {
    const int esz = elem_size(c.dtype), w = 16 / esz;
    return vec_ok(c.A, c.lda, row_len_a(c), esz, w) ? w : 1;
}
bool vec_b_ok(const Call &c, int v) { return vec_ok(c.B, c.ldb, row_len_b(c), elem_size(c.dtype), v); }

// Buffer addressing.  The kernels read operands through buffer resources
// whose byte offsets are 32-bit, with 2^31 reserved to mark a load out of
// range; each resource starts at a panel or slice of an operand (rebased as
// the kernel walks K, with 64-bit base arithmetic), so what must stay below
// 2^31 bytes is the extent of one panel or slice, not the operand:
//   - a panel of rows read whole (A stored M x K, B stored N x K): the
//     tile's valid rows, each K long rounded up to the k slice (rows past
//     them are read as the last valid one);
//   - a slice of k rows (B stored K x N, A stored K x M): tile_k rows of
//     the leading dimension, the last of them tile_n (tile_m) long;
//   - the skinny kernels: B stored K x N in batches of tile_k rows; A (16
//     rows at most) whole, or with A stored K x M as a K-row panel (fp32)
//     or per 32-row block (bf16); with B stored N x K, 32 rows of B and the
//     16 rows of A, each K long.
// The general kernels index with 64-bit element offsets and take anything.
constexpr int64_t kMaxResourceBytes = (int64_t(1) << 31) - 1;

bool panel_fits(int64_t rows, int64_t ld, int64_t row_len, int64_t esz) {
    return rows < 1 || ((rows - 1) * ld + row_len) * esz <= kMaxResourceBytes;
}

bool operands_fit(const KernelDesc *kd, const Call &c) {
    if (kd->fallback) return true;
    const int64_t esz = elem_size(c.dtype);
    const bool a_n = c.op_a == GEMM_OP_N, b_n = c.op_b == GEMM_OP_N;
    if (kd->path == GEMM_PATH_SKINNY || kd->path == GEMM_PATH_SKINNY_SPLITK) {
        if (!b_n)   // A gathered from its K x M storage when transposed: one resource over all of it
            return panel_fits(32, c.ldb, c.K, esz) && (a_n ? panel_fits(16, c.lda, c.K, esz)
                                                           : panel_fits(c.K, c.lda, c.M, esz));
        const bool b_ok = panel_fits(kd->tile_k, c.ldb, kd->tile_n, esz);
        if (a_n) return b_ok && panel_fits(c.M, c.lda, c.K, esz);
        const int64_t a_rows = c.dtype == GEMM_DTYPE_F32 ? c.K : kd->tile_k;
        return b_ok && panel_fits(a_rows, c.lda, c.M, esz);
    }
    // Rows read whole are addressed up to K rounded up to the k slice (the
    // chunks past K get 2^31 added, which must not wrap).
    const int64_t a_panel = c.M < kd->tile_m ? c.M : kd->tile_m;
    const int64_t b_panel = c.N < kd->tile_n ? c.N : kd->tile_n;
    const int64_t k_pad = ceil_div(c.K, kd->tile_k) * kd->tile_k;
    const bool a_ok = a_n ? panel_fits(a_panel, c.lda, k_pad, esz) : panel_fits(kd->tile_k, c.lda, kd->tile_m, esz);
    const bool b_ok = b_n ? panel_fits(kd->tile_k, c.ldb, kd->tile_n, esz) : panel_fits(b_panel, c.ldb, k_pad, esz);
    return a_ok && b_ok;
}

// The skinny kernels take M <= 16.
bool skinny_fits(const Call &c) { return c.M <= 16; }

int64_t split_workspace_bytes(const Call &c, const KernelDesc *kd) {
    const int64_t strips = ceil_div(c.N, kd->tile_n);
    return gemm::skinny_workspace_bytes((int)strips, (int)c.M, (int)c.N, (int)c.K);
}

bool kernel_runs(const KernelDesc *kd, const Call &c) {
    if (kd->dtype != c.dtype) return false;
    if (((kd->outputs >> c.out_type) & 1) == 0) return false;
    if (((kd->layouts >> (2 * c.op_a + c.op_b)) & 1) == 0) return false;
    if ((kd->path == GEMM_PATH_SKINNY || kd->path == GEMM_PATH_SKINNY_SPLITK) && !skinny_fits(c)) return false;
    if (!operands_fit(kd, c)) return false;
    if (kd->path == GEMM_PATH_SKINNY_SPLITK) {
        const int64_t need = split_workspace_bytes(c, kd);
        if (need > 0 && (c.ws == nullptr || c.ws_bytes < need)) return false;
    }
    if (kd->vec_a > 1 && max_vec_a(c) < kd->vec_a) return false;
    return vec_b_ok(c, kd->vec_b);
}

// K split of the tiled kernels ("Tiled matrix multiplication", "Variants and
// alternatives"; "A GEMM Kernel, Step by Step", "What is left"): when a
// problem has fewer output tiles than compute units and a deep K, the k
// range is cut into up to kMaxKSplits slices of at least kMinSplitDepth
// (whole multiples of kSplitAlign, which keeps every slice's operand bases
// 16-byte aligned); each slice's partial product goes to the caller's
// workspace and a reduce kernel adds them in order.
constexpr int kMaxKSplits = 16;
static_assert(kMaxKSplits <= gemm::kMaxReduceSplits, "the reduce kernel adds at most kMaxReduceSplits slices");
constexpr int64_t kMinSplitDepth = 1024;
constexpr int64_t kSplitAlign = 64;

struct KSplit {
    int splits;        // 1: no split
    int32_t kchunk;    // k depth of each slice (the last one may be shorter)
    int64_t bytes;     // workspace: splits partial products of the split rows
    // Rows [0, m_top) run first without a split (whole waves of tiles); the
    // split covers rows [m_top, M).  0: the split covers the whole call.
    int64_t m_top = 0;
};

KSplit tiled_ksplit(const Call &c, int tile_m, int tile_n) {
    KSplit r{1, 0, 0};
    const int64_t tiles = ceil_div(c.M, tile_m) * ceil_div(c.N, tile_n);
    int s = 1;
    while (s < kMaxKSplits && tiles * s * 2 <= kComputeUnits && c.K / (2 * s) >= kMinSplitDepth) s *= 2;
    if (s == 1) return r;
    const int64_t chunk = ceil_div(ceil_div(c.K, s), kSplitAlign) * kSplitAlign;
    r.splits = (int)ceil_div(c.K, chunk);
    if (r.splits < 2) return KSplit{1, 0, 0};
    r.kchunk = (int32_t)chunk;
    r.bytes = (int64_t)r.splits * c.M * c.N * 4;
    return r;
}

// The last, mostly empty wave ("A GEMM Kernel, Step by Step", "The fringe
// and the last wave"; the goal of Stream-K in "Tiled matrix
// multiplication", "Variants and alternatives": give every compute unit an
// equal share of the multiply-adds).  When the tile count is just over a
// multiple of the compute units, the top rows of tiles that fill whole waves
// run as usual and the few tile rows left over run as a separate K-split
// problem, whose slices spread their multiply-adds over the compute units
// that would otherwise idle.  Estimated in full-tile times: taken when it
// saves at least half of one.  Only for 256^2 tiles, one workgroup per
// compute unit: smaller tiles run two or more to a compute unit, so a wave
// holds more of them than this count assumes.
KSplit wave_tail(const Call &c, int tile) {
    const KSplit none{1, 0, 0};
    if (tile != 256) return none;
    const int64_t tiles_m = ceil_div(c.M, tile), tiles_n = ceil_div(c.N, tile);
    const int64_t T = tiles_m * tiles_n, waves = T / kComputeUnits, r = T % kComputeUnits;
    if (waves == 0 || r == 0 || 2 * r > kComputeUnits) return none;
    const int64_t dm = waves * kComputeUnits / tiles_n;       // tile rows in whole waves
    if (dm <= 0 || dm >= tiles_m) return none;
    Call bot = c;
    bot.M = c.M - dm * tile;
    KSplit ks = tiled_ksplit(bot, tile, tile);
    if (ks.splits < 2) return none;
    const int64_t bot_tiles = (tiles_m - dm) * tiles_n;
    const double plain = (double)ceil_div(T, kComputeUnits);
    const double split = (double)ceil_div(dm * tiles_n, kComputeUnits) +
                         (double)ceil_div(bot_tiles * ks.splits, kComputeUnits) / ks.splits;
    if (split > plain - 0.5) return none;
    ks.m_top = dm * tile;
    return ks;
}

// The split a tiled kernel takes for this call: none without a workspace
// large enough for it.
KSplit call_ksplit(const Call &c, const KernelDesc *kd) {
    if (kd->path != GEMM_PATH_TILED || c.ws == nullptr) return KSplit{1, 0, 0};
    KSplit r = tiled_ksplit(c, kd->tile_m, kd->tile_n);
    if (r.splits < 2) r = wave_tail(c, kd->tile_m);
    return r.splits > 1 && c.ws_bytes >= r.bytes ? r : KSplit{1, 0, 0};
}

const KernelDesc *first_match(const KernelDesc *table, int count, const Call &c, int tile_m) {
    for (int i = 0; i < count; ++i)
        if ((tile_m == 0 || table[i].tile_m == tile_m) && c.K >= table[i].min_k && kernel_runs(&table[i], c))
            return &table[i];
    return nullptr;
}

// The tiled kernels of the call's operand type that run its layout, in
// table order (which is preference order), fallback kernels or not.
struct Candidates {
    const KernelDesc *k[64];
    int n = 0;
    bool use_min_k = true;     // honour each kernel's K minimum
};
Candidates tiled_candidates(const Call &c, bool fallback) {
    Candidates r;
    for (int32_t id = 1; id <= table_size() && r.n < 64; ++id) {
        const KernelDesc *kd = kernel_by_id(id);
        if (kd->path == GEMM_PATH_TILED && kd->dtype == c.dtype && kd->fallback == fallback &&
            ((kd->layouts >> (2 * c.op_a + c.op_b)) & 1))
            r.k[r.n++] = kd;
    }
    return r;
}
const KernelDesc *first_candidate(const Candidates &cand, const Call &c, int tile_m) {
    for (int i = 0; i < cand.n; ++i)
        if ((tile_m == 0 || cand.k[i]->tile_m == tile_m) && (!cand.use_min_k || c.K >= cand.k[i]->min_k) &&
            kernel_runs(cand.k[i], c))
            return cand.k[i];
    return nullptr;
}

// Tile choice among kernels of one class (see below).
const KernelDesc *choose_tiled(const Call &c, const Candidates &cand);

// 128^2 tiles in place of 256^2 ones whose last wave is mostly empty ("A
// GEMM Kernel, Step by Step", "The fringe and the last wave").  Two 128^2
// workgroups share a compute unit and each holds a quarter of the work, so
// their last wave is eight times finer.  What the small tile gives up per
// multiply-add decides how empty the 256^2 wave must be (measured against
// 256^2 tiles unsplit):
// - the fp32 rings and the fp8 rings lose little: 128^2 tiles win once a
//   quarter of the last wave is empty (fp32 0.65-0.90 of the time, fp8
//   0.74-0.98), and the fp8 rings also win on whole waves with K <= 2048
//   (0.77-0.92), where the 256^2 ring's fill and drain weigh more;
// - the bf16 and fp8 whole-line kernels lose more: 128^2 tiles win only
//   between one and two waves with at most a quarter of the second used
//   (0.84-0.89).
bool last_wave_prefers_128(const Call &c) {
    const int64_t T = ceil_div(c.M, 256) * ceil_div(c.N, 256);
    if (T < kComputeUnits) return false;
    const int64_t empty = ceil_div(T, kComputeUnits) * kComputeUnits - T;
    const bool fp8 = c.dtype == GEMM_DTYPE_FP8F32;
    const bool lines = c.dtype == GEMM_DTYPE_BF16F32 || (fp8 && c.op_a == GEMM_OP_N && c.op_b == GEMM_OP_T);
    if (lines) return T < 2 * kComputeUnits && 4 * empty >= 3 * kComputeUnits;
    return 4 * empty >= kComputeUnits || (fp8 && c.K <= 2048);
}

// Tile choice: the largest square tile whose tile count covers every compute
// unit at least once, unless 256^2 tiles leave a mostly empty last wave
// (last_wave_prefers_128); small problems fall through to the smallest tile.  The
// rule compares kernels of like speed, so it runs over the regular kernels
// first and over the fallback (general) kernels only when none of those runs
// the call.
const KernelDesc *choose(const Call &c) {
    // fp32 and bf16 with B stored K x N: the streaming kernels, for A stored
    // either way (the table's layouts pick the A load).  The split-K kernels pay
    // off only where K is actually split.
    const bool b_kn = c.op_b == GEMM_OP_N;
    if (b_kn && c.dtype == GEMM_DTYPE_F32 && skinny_fits(c) && c.ws != nullptr) {
        const KernelDesc *kd = first_match(gemm::kF32SplitKernels, gemm::kF32SplitKernelCount, c, 0);
        if (kd != nullptr && split_workspace_bytes(c, kd) > 0) return kd;
    }
    if (b_kn && c.dtype == GEMM_DTYPE_F32 && skinny_fits(c)) {
        if (const KernelDesc *kd = first_match(gemm::kF32SkinnyKernels, gemm::kF32SkinnyKernelCount, c, 0))
            return kd;
    }
    // bf16 weights with M <= 16: the streaming kernel, split over K when the
    // caller's workspace allows (it needs one only when it splits).
    if (b_kn && c.dtype == GEMM_DTYPE_BF16F32 && skinny_fits(c)) {
        if (const KernelDesc *kd = first_match(gemm::kBf16SplitKernels, gemm::kBf16SplitKernelCount, c, 0))
            return kd;
    }
    // fp8 weights stored K x N with M <= 16: the same kernel through
    // byte-transposing reads, but only without a workspace and with at most
    // half as many 128-column strips as compute units.  With a workspace the
    // 128^2 ring split over K is as fast or faster (16 x 8192 x 8192: 18.8
    // against 19.2 us; 16 x 28672 x 4096: 22.0 against 29.9 us), and so is the
    // unsplit 128^2 ring once the strips would fill the compute units at one
    // workgroup each (16 x 28672 x 4096: 21.8 against 24.7 us).  The split
    // form stays a candidate for forced calls and the autotuner.  With A
    // stored K x M the kernel loads A a byte a lane, and runs where the
    // 128^2 ring cannot (A's K rows not whole 16-byte chunks), which left
    // only the general kernel.
    if (b_kn && c.dtype == GEMM_DTYPE_FP8F32 && skinny_fits(c)) {
        const bool ring_runs = c.op_a == GEMM_OP_N || max_vec_a(c) >= 16;
        const bool few_strips = 2 * ceil_div(c.N, gemm::kFp8SkinnyKernels[0].tile_n) <= kComputeUnits;
        if (!ring_runs || (c.op_a == GEMM_OP_N && c.ws == nullptr && few_strips)) {
            if (const KernelDesc *kd = first_match(gemm::kFp8SkinnyKernels, gemm::kFp8SkinnyKernelCount, c, 0))
                return kd;
        }
    }
    // M <= 16 with B stored N x K (a linear layer's weights): the streaming
    // kernel that reads weight rows straight into the matrix instruction,
    // split over K only where the workspace lets it cover the compute units.
    // With A stored K x M as well, the same kernel gathers A element by
    // element (16 x 8192 x 8192: fp32 60 us against 98-168 us on the rings,
    // bf16 37 against 41-148 us), except fp8 with a workspace where the 128^2
    // ring can run: split over K it takes 18.3 us against 26.0 us.
    const bool fp8_tt_ring = c.op_a == GEMM_OP_T && c.dtype == GEMM_DTYPE_FP8F32 && c.ws != nullptr &&
                             max_vec_a(c) >= 16;
    if (c.op_b == GEMM_OP_T && skinny_fits(c) && !fp8_tt_ring) {   // A stored either way (the layouts pick)
        for (int i = 0; i < gemm::kSkinnyNtKernelCount; ++i) {
            const KernelDesc *kd = &gemm::kSkinnyNtKernels[i];
            if (kd->path == GEMM_PATH_SKINNY_SPLITK && c.ws != nullptr && split_workspace_bytes(c, kd) > 0 &&
                kernel_runs(kd, c))
                return kd;
        }
        for (int i = 0; i < gemm::kSkinnyNtKernelCount; ++i) {
            const KernelDesc *kd = &gemm::kSkinnyNtKernels[i];
            if (kd->path == GEMM_PATH_SKINNY && kernel_runs(kd, c)) return kd;
        }
    }
    Candidates regular = tiled_candidates(c, false);
    if (const KernelDesc *kd = choose_tiled(c, regular)) return kd;
    // A K minimum prefers another regular kernel for short K; where none of
    // those runs the call (say, an output type they cannot write), the
    // kernel is still better than a fallback.
    regular.use_min_k = false;
    if (const KernelDesc *kd = choose_tiled(c, regular)) return kd;
    return choose_tiled(c, tiled_candidates(c, true));
}

const KernelDesc *choose_tiled(const Call &c, const Candidates &cand) {
    // With a workspace: the largest tile that wastes at most a quarter of
    // its padded M x N ("The fringe and the last wave": tile quantisation)
    // and whose grid of tiles x K slices fills at least three quarters of the
    // compute units.  Padding costs the fp32 kernels 8x more time than the
    // bf16 ones (their matrix rate is 8x lower), so thin problems go to small
    // tiles even when a large tile would have enough slices.
    // A tile left unsplit must still fill a whole wave, as in the rule
    // below (fp32 1000 x 3000 x 777: 752 tiles of 64^2 take 60 us, the 192
    // of 128^2 that fill three quarters of the compute units 95 us).
    if (c.ws != nullptr) {
        for (int tile : {256, 128, 64}) {
            const KernelDesc *kd = first_candidate(cand, c, tile);
            if (kd == nullptr) continue;
            const int64_t pm = ceil_div(c.M, tile) * tile, pn = ceil_div(c.N, tile) * tile;
            const KSplit ks = call_ksplit(c, kd);
            const int64_t groups = (pm / tile) * (pn / tile) * ks.splits;
            const bool fills = ks.splits > 1 ? 4 * groups >= 3 * kComputeUnits : groups >= kComputeUnits;
            // A split sends every partial product through the workspace and
            // back (2048 x 4096 x 4096 in two: 160 MB), which costs more than
            // 128^2 tiles give up against 256^2 ones, so 128^2 tiles that
            // fill the compute units unsplit go first (there: 68 us against
            // 87 us for 256^2 tiles in two slices in bf16, 41 against 63 us
            // in fp8, 496 against 507-549 us in fp32).  64^2 tiles lose more
            // than that to 128^2 ones, so a split 128^2 tile stays, and so
            // does a last-wave split, whose partials cover one tile row.
            if (ks.splits > 1 && ks.m_top == 0 && tile == 256 &&
                ceil_div(c.M, tile / 2) * ceil_div(c.N, tile / 2) >= kComputeUnits &&
                first_candidate(cand, c, tile / 2) != nullptr)
                continue;
            // A mostly empty last wave (above) goes to 128^2 tiles too when
            // its tile rows would run as a last-wave split, except in bf16:
            // 128^2 tiles took 0.74-0.97 of the split's time in fp8 and
            // 0.85-1.01 in fp32, but 0.91-1.10 in bf16.
            if (tile == 256 && (ks.splits == 1 || (ks.m_top > 0 && c.dtype != GEMM_DTYPE_BF16F32)) &&
                last_wave_prefers_128(c) && first_candidate(cand, c, 128) != nullptr)
                continue;
            if (4 * c.M * c.N >= 3 * pm * pn && fills) return kd;
        }
    }
    // The smallest tile among the kernels that can run the call.
    int smallest = 1 << 30;
    for (int i = 0; i < cand.n; ++i)
        if (kernel_runs(cand.k[i], c) && cand.k[i]->tile_m < smallest) smallest = cand.k[i]->tile_m;
    for (int tile : {256, 128, 64}) {
        const int64_t tiles = ceil_div(c.M, tile) * ceil_div(c.N, tile);
        if (tile == 256 && last_wave_prefers_128(c) && first_candidate(cand, c, 128) != nullptr) continue;
        if (tiles >= kComputeUnits || tile == smallest) {
            if (const KernelDesc *kd = first_candidate(cand, c, tile)) return kd;
        }
    }
    return first_candidate(cand, c, 0);
}

// Per-shape tuning ("A GEMM Kernel, Step by Step", "Six parameters, found by
// search": the best kernel for a shape is found by timing the candidates).
// gemm_autotune() times every kernel that can run a call, with and without a
// K split, and records the fastest here; calls of the same operand type,
// layout, shape, operand alignment class and workspace presence then take
// that choice whenever it still fits the call.
struct TuneKey {
    int32_t dtype;
    int32_t op_a, op_b;      // GEMM_OP_N or GEMM_OP_T
    int64_t M, N, K;
    int32_t vec_a, vec_b;    // widest vector loads A and B allow
    int32_t has_ws;
    bool operator<(const TuneKey &o) const {
        return std::tie(dtype, op_a, op_b, M, N, K, vec_a, vec_b, has_ws) <
               std::tie(o.dtype, o.op_a, o.op_b, o.M, o.N, o.K, o.vec_a, o.vec_b, o.has_ws);
    }
};
struct TuneEntry {
    int32_t kernel_id;
    int32_t split;           // 1: K split allowed (when the workspace suffices); 0: never
    float ms;                // measured time per call
};
std::mutex g_tune_mu;
std::map<TuneKey, TuneEntry> g_tuned;

int max_vec_b(const Call &c) {
    const int w = 16 / elem_size(c.dtype);
    return vec_b_ok(c, w) ? w : 1;
}

TuneKey tune_key(const Call &c) {
    return TuneKey{c.dtype, c.op_a, c.op_b, c.M, c.N, c.K, max_vec_a(c), max_vec_b(c), c.ws != nullptr ? 1 : 0};
}

// A tuned choice for this call, if one was recorded and still fits it.
bool tuned_choice(const Call &c, const KernelDesc **kd, bool *allow_split) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    auto it = g_tuned.find(tune_key(c));
    if (it == g_tuned.end()) return false;
    const KernelDesc *k = kernel_by_id(it->second.kernel_id);
    if (k == nullptr || !kernel_runs(k, c)) return false;
    *kd = k;
    *allow_split = it->second.split != 0;
    return true;
}

// The plan of a call: the kernel (forced, tuned or chosen) and its K split.
gemm_status plan(const Call &c, int32_t force, gemm_plan *out, const KernelDesc **chosen, KSplit *split,
                 bool use_tuned = true, bool allow_split = true) {
    gemm_plan pl;
    std::memset(&pl, 0, sizeof pl);
    *chosen = nullptr;
    *split = KSplit{1, 0, 0};
    gemm_status st = validate(c);
    if (st != GEMM_OK) return st;
    if (force < 0 || (force > 0 && kernel_by_id(force) == nullptr)) return GEMM_ERR_INVALID_ARG;
    if (c.M == 0 || c.N == 0) {
        pl.path = GEMM_PATH_NONE;
    } else if (c.K == 0 || c.alpha == 0.0f) {
        pl.path = GEMM_PATH_SCALE;
        pl.threads = 256;
        pl.grid = ceil_div(c.M * c.N, 256) < 4096 ? ceil_div(c.M * c.N, 256) : 4096;
    } else {
        const KernelDesc *kd = nullptr;
        if (force > 0) {
            kd = kernel_by_id(force);
        } else if (!(use_tuned && tuned_choice(c, &kd, &allow_split))) {
            kd = choose(c);
        }
        if (kd == nullptr || !kernel_runs(kd, c)) return GEMM_ERR_UNSUPPORTED;
        pl.path = kd->path;
        pl.kernel_id = id_of(kd);
        pl.threads = kd->threads;
        pl.tile_m = kd->tile_m;
        pl.tile_n = kd->tile_n;
        pl.tile_k = kd->tile_k;
        pl.vec_a = kd->vec_a;
        pl.vec_b = kd->vec_b;
        if (kd->path == GEMM_PATH_SKINNY) {
            pl.grid = ceil_div(c.N, kd->tile_n);
        } else if (kd->path == GEMM_PATH_SKINNY_SPLITK) {
            const int64_t strips = ceil_div(c.N, kd->tile_n);
            pl.grid = strips * gemm::skinny_splits((int)strips, (int)c.K);
        } else {
            if (allow_split) *split = call_ksplit(c, kd);
            pl.splits = split->splits;
            pl.split_row = split->m_top;
            const int64_t tiles_n = ceil_div(c.N, kd->tile_n);
            pl.grid = ceil_div(split->m_top, kd->tile_m) * tiles_n +
                      ceil_div(c.M - split->m_top, kd->tile_m) * tiles_n * pl.splits;
        }
        if (pl.splits == 0) pl.splits = 1;
        *chosen = kd;
    }
    if (out) *out = pl;
    return GEMM_OK;
}

// The current device must be a gfx950; checked once per device and cached.
std::atomic<int8_t> g_device_ok[64];

gemm_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_DEVICE;
    if (dev < 64) {
        const int8_t known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known != 0) return known > 0 ? GEMM_OK : GEMM_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_device_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? GEMM_OK : GEMM_ERR_DEVICE;
}

gemm_status launch(const Call &c, const gemm_plan &pl, const KernelDesc *kd, const KSplit &ks, hipStream_t s);

gemm_status run(const Call &c, int32_t force, gemm_stream_t stream) {
    gemm_plan pl;
    const KernelDesc *kd = nullptr;
    KSplit ks;
    gemm_status st = plan(c, force, &pl, &kd, &ks);
    if (st != GEMM_OK || pl.path == GEMM_PATH_NONE) return st;
    st = check_device();
    if (st != GEMM_OK) return st;
    return launch(c, pl, kd, ks, static_cast<hipStream_t>(stream));
}

gemm_status launch(const Call &c, const gemm_plan &pl, const KernelDesc *kd, const KSplit &ks, hipStream_t s) {
    gemm::GemmParams p;
    p.A = c.A;
    p.B = c.B;
    p.C = c.C;
    p.M = (int32_t)c.M;
    p.N = (int32_t)c.N;
    p.K = (int32_t)c.K;
    p.lda = (int32_t)c.lda;
    p.ldb = (int32_t)c.ldb;
    p.ldc = c.ldc;
    p.alpha = c.alpha;
    p.beta = c.beta;
    p.op_a = c.op_a;
    p.op_b = c.op_b;
    p.kchunk = 0;
    p.partials = nullptr;
    p.bias = c.bias;
    p.act = c.act;
    p.out_type = c.out_type;
    p.out_scale = c.out_scale;
    p.out = c.out_type == GEMM_OUT_F32 ? static_cast<void *>(c.C) : c.out;
    p.ldo = c.out_type == GEMM_OUT_F32 ? c.ldc : c.ldo;
    hipError_t err;
    if (pl.path == GEMM_PATH_SCALE) {
        err = gemm::launch_scale_c(p, s);
    } else if (ks.splits > 1 && ks.m_top > 0) {
        // Whole waves of the top rows, then the K-split bottom rows (A's
        // rows are its columns when it is stored transposed).
        gemm::GemmParams top = p;
        top.M = (int32_t)ks.m_top;
        err = kd->launch(top, s);
        const int64_t esz = elem_size(c.dtype);
        const int64_t a_off = (c.op_a == GEMM_OP_N ? ks.m_top * c.lda : ks.m_top) * esz;
        const int64_t out_esz = c.out_type == GEMM_OUT_F32 ? 4 : c.out_type == GEMM_OUT_BF16 ? 2 : 1;
        p.A = static_cast<const char *>(c.A) + a_off;
        if (c.C != nullptr) p.C = c.C + ks.m_top * c.ldc;
        p.out = static_cast<char *>(p.out) + ks.m_top * p.ldo * out_esz;
        p.M = (int32_t)(c.M - ks.m_top);
        p.kchunk = ks.kchunk;
        p.partials = static_cast<float *>(c.ws);
        if (err == hipSuccess) err = kd->launch(p, s);
        if (err == hipSuccess) err = gemm::launch_splitk_reduce(p, s);
    } else if (ks.splits > 1) {
        p.kchunk = ks.kchunk;
        p.partials = static_cast<float *>(c.ws);
        err = kd->launch(p, s);
        if (err == hipSuccess) err = gemm::launch_splitk_reduce(p, s);
    } else {
        err = kd->launch_ws ? kd->launch_ws(p, c.ws, s) : kd->launch(p, s);
    }
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// Mean time of `reps` calls of one candidate (after one untimed call), by
// HIP events on the call's stream.  GEMM_ERR_UNSUPPORTED if it cannot run.
gemm_status time_candidate(const Call &c, const KernelDesc *kd, bool allow_split, int reps, hipStream_t s,
                           float *ms, bool *split_used) {
    gemm_plan pl;
    const KernelDesc *k = nullptr;
    KSplit ks;
    gemm_status st = plan(c, id_of(kd), &pl, &k, &ks, false, allow_split);
    if (st != GEMM_OK) return st;
    *split_used = ks.splits > 1;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return GEMM_ERR_LAUNCH;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return GEMM_ERR_LAUNCH;
    }
    st = launch(c, pl, k, ks, s);
    if (st == GEMM_OK && hipEventRecord(e0, s) != hipSuccess) st = GEMM_ERR_LAUNCH;
    for (int r = 0; st == GEMM_OK && r < reps; ++r) st = launch(c, pl, k, ks, s);
    if (st == GEMM_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess))
        st = GEMM_ERR_LAUNCH;
    float total = 0.0f;
    if (st == GEMM_OK && hipEventElapsedTime(&total, e0, e1) != hipSuccess) st = GEMM_ERR_LAUNCH;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms = total / (float)reps;
    return st;
}

gemm_status autotune(const Call &c, int reps, hipStream_t s, gemm_plan *out) {
    if (reps < 1 || reps > 1000 || out == nullptr) return GEMM_ERR_INVALID_ARG;
    const KernelDesc *kd = nullptr;
    KSplit ks;
    gemm_status st = plan(c, 0, out, &kd, &ks, false);
    if (st != GEMM_OK || out->path == GEMM_PATH_NONE || out->path == GEMM_PATH_SCALE) return st;
    st = check_device();
    if (st != GEMM_OK) return st;
    TuneEntry best{0, 0, 0.0f};
    for (int32_t id = 1; id <= table_size(); ++id) {
        const KernelDesc *cand = kernel_by_id(id);
        if (cand->dtype != c.dtype || !kernel_runs(cand, c)) continue;
        for (int split = 0; split < 2; ++split) {
            float ms = 0.0f;
            bool used = false;
            st = time_candidate(c, cand, split == 1, reps, s, &ms, &used);
            if (st == GEMM_ERR_UNSUPPORTED) break;
            if (st != GEMM_OK) return st;
            if (split == 1 && !used) break;            // no split possible: same as the first timing
            if (best.kernel_id == 0 || ms < best.ms) best = TuneEntry{id, split, ms};
        }
    }
    if (best.kernel_id == 0) return GEMM_ERR_UNSUPPORTED;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        g_tuned[tune_key(c)] = best;
    }
    return plan(c, 0, out, &kd, &ks);
}

Call make_call(int32_t dtype, int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
               const void *B, int64_t ldb, float beta, const float *C, int64_t ldc, void *ws = nullptr,
               int64_t ws_bytes = 0) {
    Call c;
    c.ws = ws;
    c.ws_bytes = ws ? ws_bytes : 0;
    c.bias = nullptr;
    c.act = GEMM_ACT_NONE;
    c.out_type = GEMM_OUT_F32;
    c.out = nullptr;
    c.ldo = 0;
    c.out_scale = 1.0f;
    c.dtype = dtype;
    c.op_a = GEMM_OP_N;
    c.op_b = GEMM_OP_N;
    c.M = M;
    c.N = N;
    c.K = K;
    c.alpha = alpha;
    c.beta = beta;
    c.A = A;
    c.B = B;
    c.C = const_cast<float *>(C);
    c.lda = lda;
    c.ldb = ldb;
    c.ldc = ldc;
    return c;
}

// The operand layouts of a call.  A single row of A stored transposed (K x 1)
// with unit leading dimension is the same memory as that row stored M x K, so
// unless a kernel is forced it runs as one: the M <= 16 streaming kernels
// then take it, whatever its alignment along M (which is what keeps them from
// A stored K x M).
void set_ops(Call &c, int32_t op_a, int32_t op_b, int32_t force_kernel = 0) {
    c.op_a = op_a;
    c.op_b = op_b;
    if (force_kernel == 0 && op_a == GEMM_OP_T && c.M == 1 && c.lda == 1) {
        c.op_a = GEMM_OP_N;
        c.lda = c.K > 1 ? c.K : 1;
    }
}

}  // namespace

extern "C" {

GEMM_API gemm_status gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                              const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                              gemm_stream_t stream) {
    return run(make_call(GEMM_DTYPE_F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), 0, stream);
}

GEMM_API gemm_status gemm_bf16f32(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                  int64_t lda, const uint16_t *B, int64_t ldb, float beta, float *C,
                                  int64_t ldc, gemm_stream_t stream) {
    return run(make_call(GEMM_DTYPE_BF16F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), 0, stream);
}

GEMM_API gemm_status gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                                 const float *B, int64_t ldb, float beta, float *C, int64_t ldc, void *workspace,
                                 int64_t workspace_bytes, gemm_stream_t stream) {
    return run(make_call(GEMM_DTYPE_F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes),
               0, stream);
}

GEMM_API gemm_status gemm_bf16f32_ws(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                     int64_t lda, const uint16_t *B, int64_t ldb, float beta, float *C,
                                     int64_t ldc, void *workspace, int64_t workspace_bytes, gemm_stream_t stream) {
    return run(make_call(GEMM_DTYPE_BF16F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                         workspace_bytes),
               0, stream);
}

}  // extern "C"

namespace {

// Calls with a fused epilogue; a NULL descriptor is the plain call.
void apply_epilogue(Call &c, const gemm_epilogue *epi) {
    if (epi == nullptr) return;
    c.bias = epi->bias;
    c.act = epi->activation;
    c.out_type = epi->out_type;
    c.out = epi->out;
    c.ldo = epi->ldo;
    c.out_scale = epi->out_scale == 0.0f ? 1.0f : epi->out_scale;
}

gemm_status run_epi(Call c, const gemm_epilogue *epi, int32_t force, gemm_stream_t stream) {
    apply_epilogue(c, epi);
    return run(c, force, stream);
}

}  // namespace

extern "C" {

GEMM_API gemm_status gemm_f32_epi(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                                  const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                                  const gemm_epilogue *epilogue, void *workspace, int64_t workspace_bytes,
                                  gemm_stream_t stream) {
    return run_epi(make_call(GEMM_DTYPE_F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                             workspace_bytes),
                   epilogue, 0, stream);
}

GEMM_API gemm_status gemm_bf16f32_epi(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                      int64_t lda, const uint16_t *B, int64_t ldb, float beta, float *C,
                                      int64_t ldc, const gemm_epilogue *epilogue, void *workspace,
                                      int64_t workspace_bytes, gemm_stream_t stream) {
    return run_epi(make_call(GEMM_DTYPE_BF16F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                             workspace_bytes),
                   epilogue, 0, stream);
}

GEMM_API gemm_status gemm_f32_ex(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
                                 const float *B, int64_t ldb, float beta, float *C, int64_t ldc,
                                 int32_t force_kernel, const gemm_epilogue *epilogue, void *workspace,
                                 int64_t workspace_bytes, gemm_stream_t stream) {
    return run_epi(make_call(GEMM_DTYPE_F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                             workspace_bytes),
                   epilogue, force_kernel, stream);
}

GEMM_API int64_t gemm_workspace_size(int32_t dtype, int64_t M, int64_t N, int64_t K) {
    if ((dtype != GEMM_DTYPE_F32 && dtype != GEMM_DTYPE_BF16F32 && dtype != GEMM_DTYPE_FP8F32) || M <= 0 ||
        N <= 0 || K <= 0 ||
        M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return 0;
    int64_t need = 0;
    // Tiled K split: the largest tile gives the most slices.
    Call c = make_call(dtype, M, N, K, 1.0f, nullptr, K, nullptr, N, 0.0f, nullptr, N);
    for (int tile : {256, 128, 64}) {
        const KSplit ks = tiled_ksplit(c, tile, tile);
        need = ks.bytes > need ? ks.bytes : need;
        const KSplit tail = wave_tail(c, tile);
        need = tail.bytes > need ? tail.bytes : need;
    }
    if (M > 16) return need;
    const gemm::KernelDesc *skinny = dtype == GEMM_DTYPE_F32       ? gemm::kF32SplitKernels
                                     : dtype == GEMM_DTYPE_BF16F32 ? gemm::kBf16SplitKernels
                                                                   : gemm::kFp8SkinnyKernels;
    const int count = dtype == GEMM_DTYPE_F32       ? gemm::kF32SplitKernelCount
                      : dtype == GEMM_DTYPE_BF16F32 ? gemm::kBf16SplitKernelCount
                                                    : gemm::kFp8SkinnyKernelCount;
    for (int i = 0; i < count; ++i) {
        const int64_t strips = ceil_div(N, skinny[i].tile_n);
        const int64_t b = gemm::skinny_workspace_bytes((int)strips, (int)M, (int)N, (int)K);
        need = b > need ? b : need;
    }
    for (int i = 0; i < gemm::kSkinnyNtKernelCount; ++i) {
        const gemm::KernelDesc &kd = gemm::kSkinnyNtKernels[i];
        if (kd.dtype != dtype || kd.path != GEMM_PATH_SKINNY_SPLITK) continue;
        const int64_t strips = ceil_div(N, kd.tile_n);
        const int64_t b = gemm::skinny_workspace_bytes((int)strips, (int)M, (int)N, (int)K);
        need = b > need ? b : need;
    }
    return need;
}

GEMM_API gemm_status gemm_bf16f32_ex(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t *A,
                                     int64_t lda, const uint16_t *B, int64_t ldb, float beta, float *C,
                                     int64_t ldc, int32_t force_kernel, const gemm_epilogue *epilogue,
                                     void *workspace, int64_t workspace_bytes, gemm_stream_t stream) {
    return run_epi(make_call(GEMM_DTYPE_BF16F32, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                             workspace_bytes),
                   epilogue, force_kernel, stream);
}

GEMM_API gemm_status gemm_general(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N, int64_t K,
                                  float alpha, const void *A, int64_t lda, const void *B, int64_t ldb, float beta,
                                  float *C, int64_t ldc, int32_t force_kernel, const gemm_epilogue *epilogue,
                                  void *workspace, int64_t workspace_bytes, gemm_stream_t stream) {
    Call c = make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes);
    set_ops(c, op_a, op_b, force_kernel);
    return run_epi(c, epilogue, force_kernel, stream);
}

GEMM_API gemm_status gemm_general_noalloc(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N,
                                          int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                                          int64_t ldb, float beta, float *C, int64_t ldc, int32_t force_kernel,
                                          const gemm_epilogue *epilogue, gemm_stream_t stream) {
    static_assert(gemm::kStaticScratchBytes == GEMM_STATIC_SCRATCH_BYTES, "header and library disagree");
    Call c = make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    set_ops(c, op_a, op_b, force_kernel);
    apply_epilogue(c, epilogue);
    // Argument errors first, with no HIP call, exactly as gemm_general.
    {
        gemm_plan pl;
        const KernelDesc *kd = nullptr;
        KSplit ks;
        const gemm_status st = plan(c, force_kernel, &pl, &kd, &ks);
        if (st != GEMM_OK || pl.path == GEMM_PATH_NONE) return st;
    }
    if (gemm_workspace_size(dtype, M, N, K) > gemm::kStaticScratchBytes) return GEMM_ERR_SCRATCH;
    gemm_status st = check_device();
    if (st != GEMM_OK) return st;
    void *scratch = nullptr;
    if (gemm::static_scratch(&scratch) != hipSuccess) return GEMM_ERR_DEVICE;
    c.ws = scratch;
    c.ws_bytes = gemm::kStaticScratchBytes;
    return run(c, force_kernel, stream);
}

GEMM_API gemm_status gemm_plan_query_epi(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N,
                                         int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                                         int64_t ldb, float beta, const float *C, int64_t ldc, int32_t force_kernel,
                                         const gemm_epilogue *epilogue, int64_t workspace_bytes, gemm_plan *out) {
    if (out == nullptr) return GEMM_ERR_INVALID_ARG;
    const KernelDesc *kd = nullptr;
    void *ws = workspace_bytes > 0 ? reinterpret_cast<void *>(uintptr_t(256)) : nullptr;
    Call c = make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws, workspace_bytes);
    set_ops(c, op_a, op_b, force_kernel);
    apply_epilogue(c, epilogue);
    KSplit ks;
    return plan(c, force_kernel, out, &kd, &ks);
}

GEMM_API gemm_status gemm_plan_query_general(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N,
                                             int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                                             int64_t ldb, float beta, const float *C, int64_t ldc,
                                             int32_t force_kernel, int64_t workspace_bytes, gemm_plan *out) {
    return gemm_plan_query_epi(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, force_kernel, nullptr,
                               workspace_bytes, out);
}


GEMM_API gemm_status gemm_plan_query(int32_t dtype, int64_t M, int64_t N, int64_t K, float alpha,
                                     const void *A, int64_t lda, const void *B, int64_t ldb, float beta,
                                     const float *C, int64_t ldc, int32_t force_kernel, int64_t workspace_bytes,
                                     gemm_plan *out) {
    if (out == nullptr) return GEMM_ERR_INVALID_ARG;
    const KernelDesc *kd = nullptr;
    // Planning never touches the workspace; a non-null stand-in marks that one is passed.
    void *ws = workspace_bytes > 0 ? reinterpret_cast<void *>(uintptr_t(256)) : nullptr;
    KSplit ks;
    return plan(make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws, workspace_bytes), force_kernel,
                out, &kd, &ks);
}

GEMM_API gemm_status gemm_autotune(int32_t dtype, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                   int64_t lda, const void *B, int64_t ldb, float beta, float *C, int64_t ldc,
                                   void *workspace, int64_t workspace_bytes, int32_t reps, gemm_stream_t stream,
                                   gemm_plan *out) {
    return autotune(make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes),
                    reps, static_cast<hipStream_t>(stream), out);
}

GEMM_API gemm_status gemm_autotune_general(int32_t dtype, int32_t op_a, int32_t op_b, int64_t M, int64_t N,
                                           int64_t K, float alpha, const void *A, int64_t lda, const void *B,
                                           int64_t ldb, float beta, float *C, int64_t ldc, void *workspace,
                                           int64_t workspace_bytes, int32_t reps, gemm_stream_t stream,
                                           gemm_plan *out) {
    Call c = make_call(dtype, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes);
    set_ops(c, op_a, op_b);
    return autotune(c, reps, static_cast<hipStream_t>(stream), out);
}

GEMM_API int32_t gemm_tuning_count(void) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    return (int32_t)g_tuned.size();
}

GEMM_API void gemm_tuning_clear(void) {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned.clear();
}

// One line per entry: dtype op_a op_b M N K vec_a vec_b has_workspace
// kernel_name split ms (format v2; v1 files, written before layouts were
// tuned, lack op_a op_b and load as untransposed entries).  Kernels are
// named, not numbered, so a table survives a reordered kernel list.
GEMM_API gemm_status gemm_tuning_save(const char *path) {
    if (path == nullptr) return GEMM_ERR_INVALID_ARG;
    std::FILE *f = std::fopen(path, "w");
    if (f == nullptr) return GEMM_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_tune_mu);
    bool ok =
        std::fprintf(f, "# libgemm tuning table v2: dtype op_a op_b M N K vec_a vec_b has_ws kernel split ms\n") > 0;
    for (const auto &kv : g_tuned) {
        const TuneKey &k = kv.first;
        const KernelDesc *kd = kernel_by_id(kv.second.kernel_id);
        ok = ok && kd != nullptr &&
             std::fprintf(f, "%d %d %d %lld %lld %lld %d %d %d %s %d %.6f\n", k.dtype, k.op_a, k.op_b,
                          (long long)k.M, (long long)k.N, (long long)k.K, k.vec_a, k.vec_b, k.has_ws, kd->name,
                          kv.second.split, (double)kv.second.ms) > 0;
    }
    ok = (std::fclose(f) == 0) && ok;
    return ok ? GEMM_OK : GEMM_ERR_INVALID_ARG;
}

GEMM_API int32_t gemm_tuning_load(const char *path) {
    if (path == nullptr) return -1;
    std::FILE *f = std::fopen(path, "r");
    if (f == nullptr) return -1;
    std::vector<std::pair<TuneKey, TuneEntry>> rows;
    char line[512];
    bool ok = true;
    bool v2 = false;
    while (ok && std::fgets(line, sizeof line, f) != nullptr) {
        if (std::strncmp(line, "# libgemm tuning table v2", 25) == 0) v2 = true;
        if (line[0] == '#' || line[0] == '\n') continue;
        TuneKey k;
        long long M, N, K;
        char name[128];
        int split;
        double ms;
        k.op_a = k.op_b = GEMM_OP_N;
        const int got =
            v2 ? std::sscanf(line, "%d %d %d %lld %lld %lld %d %d %d %127s %d %lf", &k.dtype, &k.op_a, &k.op_b, &M,
                             &N, &K, &k.vec_a, &k.vec_b, &k.has_ws, name, &split, &ms)
               : std::sscanf(line, "%d %lld %lld %lld %d %d %d %127s %d %lf", &k.dtype, &M, &N, &K, &k.vec_a,
                             &k.vec_b, &k.has_ws, name, &split, &ms);
        if (got != (v2 ? 12 : 10) || (k.op_a != GEMM_OP_N && k.op_a != GEMM_OP_T) ||
            (k.op_b != GEMM_OP_N && k.op_b != GEMM_OP_T)) {
            ok = false;
            break;
        }
        k.M = M;
        k.N = N;
        k.K = K;
        int32_t id = 0;
        for (int32_t i = 1; i <= table_size(); ++i)
            if (std::strcmp(kernel_by_id(i)->name, name) == 0) id = i;
        // An unknown kernel, or one for another operand type or layout: skip.
        if (id == 0 || kernel_by_id(id)->dtype != k.dtype ||
            ((kernel_by_id(id)->layouts >> (2 * k.op_a + k.op_b)) & 1) == 0)
            continue;
        rows.push_back({k, TuneEntry{id, split != 0 ? 1 : 0, (float)ms}});
    }
    std::fclose(f);
    if (!ok) return -1;
    std::lock_guard<std::mutex> lock(g_tune_mu);
    for (const auto &r : rows) g_tuned[r.first] = r.second;
    return (int32_t)rows.size();
}

GEMM_API int32_t gemm_kernel_count(void) { return table_size(); }

GEMM_API gemm_status gemm_kernel_query(int32_t id, gemm_kernel_info *out) {
    const KernelDesc *kd = kernel_by_id(id);
    if (kd == nullptr || out == nullptr) return GEMM_ERR_INVALID_ARG;
    out->id = id;
    out->dtype = kd->dtype;
    out->path = kd->path;
    out->tile_m = kd->tile_m;
    out->tile_n = kd->tile_n;
    out->tile_k = kd->tile_k;
    out->threads = kd->threads;
    out->vec_a = kd->vec_a;
    out->vec_b = kd->vec_b;
    out->name = kd->name;
    out->outputs = kd->outputs;
    out->layouts = kd->layouts;
    return GEMM_OK;
}

GEMM_API const char *gemm_status_string(gemm_status status) {
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_ARG: return "invalid argument (size, leading dimension or pointer)";
    case GEMM_ERR_UNSUPPORTED: return "unsupported problem or kernel for these operands";
    case GEMM_ERR_LAUNCH: return "HIP kernel launch failed";
    case GEMM_ERR_DEVICE: return "no usable gfx950 device is current";
    case GEMM_ERR_SCRATCH: return "the problem's K split could need more than the library's static scratch";
    }
    return "unknown status";
}

}  // extern "C"
