// Device helpers shared by the libgemm kernels (gfx950 only).
//
// Global memory is read through raw buffer loads.  A buffer resource carries
// a base address and a byte extent; the hardware returns zero for any access
// at or beyond the extent instead of touching memory.  That gives the
// zero-filled edge tiles of the blocked method ("GEMM Worklog I", section 3,
// and the "Code" section of "Tiled matrix multiplication": out-of-range
// operand elements load as 0) without a branch per element: rows past the
// end of an operand fall outside the extent, and the few lanes that must be
// masked inside it (the K tail of A) get an offset that is always outside.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"
#include "gemm_kernels.hpp"

namespace gemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family
// parts: 32-bit data format, range checked against num_records in bytes.
constexpr uint32_t kBufferWord3 = 0x00020000u;

// Extents are kept below 2^31 bytes, so this offset is always out of range.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kMaxExtent = 0x7fffffffu;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)bytes, (int)kBufferWord3);
}

__device__ __forceinline__ uint32_t clamp_extent(int64_t bytes) {
    return bytes <= 0 ? 0u : (bytes > (int64_t)kMaxExtent ? kMaxExtent : (uint32_t)bytes);
}

// Byte offset of element (row, col) of an operand panel whose buffer
// resource starts at the panel's first row and ends after its last valid row
// (`rows` of them, rows >= 1).  A row past the last valid one is read as that
// row instead: such rows only feed outputs that are never stored, and the
// clamp keeps every offset inside the panel, whose extent the host checks to
// be below 2^31 bytes, however large the leading dimension.
__device__ __forceinline__ uint32_t panel_off(int row, int rows, int ld, int col, int esz) {
    return (uint32_t)(min(row, rows - 1) * ld + col) * (uint32_t)esz;
}

__device__ __forceinline__ u32x4 load_b128(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 load_b64(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t load_b32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// Non-temporal ("nt" cache-policy bit) variants for data read exactly once.
// Streaming such data through the caches with the normal policy displaces
// whatever else they hold; in particular a large C just written by a
// previous kernel then gets written back to HBM while this kernel runs.
constexpr int kCpolNonTemporal = 2;
__device__ __forceinline__ u32x4 load_b128_nt(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNonTemporal));
}
__device__ __forceinline__ u32x2 load_b64_nt(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolNonTemporal));
}
__device__ __forceinline__ uint32_t load_b32_nt(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCpolNonTemporal);
}
__device__ __forceinline__ uint16_t load_b16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Map a hardware workgroup id to a (tile row, tile column) of C.
//
// Two orderings are composed.  (1) The dispatcher hands consecutive
// workgroup ids to the 8 XCDs in turn, and each XCD has its own L2, so the
// ids are first regrouped so that each XCD owns a contiguous range of
// logical tiles.  (2) Logical tiles are then walked in column-major order
// inside bands of `group_m` tile rows, so the tiles resident together on an
// XCD share a few A row panels and B column panels in its L2 -- the
// swizzled block order "Tiled matrix multiplication" recommends for L2
// reuse ("Complexity and constants").
__host__ __device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int group_m,
                                                     int &tm, int &tn) {
    const int total = tiles_m * tiles_n;
    const int per_xcd = total >> 3;
    int w = wg;
    if (wg < (per_xcd << 3)) w = (wg & 7) * per_xcd + (wg >> 3);
    const int band = group_m * tiles_n;
    const int g = w / band;
    const int first = g * group_m;
    const int rows = tiles_m - first < group_m ? tiles_m - first : group_m;
    const int r = w - g * band;
    tm = first + r % rows;
    tn = r / rows;
}

// Map a workgroup id to a tile for grids whose tile counts are multiples of
// 16 (otherwise fall back to tile_coords).  The 256 workgroups resident at
// once (one per compute unit) are given one 16 x 16-tile square of C, so the
// operand panels live in the shared last-level cache at any moment are those
// of 16 tile rows and 16 tile columns rather than of a whole dimension;
// squares are visited in a snake so consecutive rounds share half their
// panels.  Inside a square, hardware id w runs on XCD w % 8, which takes a
// 4 x 8 block of tiles so its 32 compute units share 4 A panels and 8 B
// panels in that XCD's L2.
__host__ __device__ __forceinline__ void tile_coords_square(int wg, int tiles_m, int tiles_n, int group_m,
                                                            int &tm, int &tn) {
    if ((tiles_m & 15) || (tiles_n & 15)) {
        tile_coords(wg, tiles_m, tiles_n, group_m, tm, tn);
        return;
    }
    const int round = wg >> 8, slot = wg & 255;
    const int squares_n = tiles_n >> 4;
    const int sq_r = round / squares_n;
    int sq_c = round - sq_r * squares_n;
    if (sq_r & 1) sq_c = squares_n - 1 - sq_c;
    const int xcd = slot & 7, j = slot >> 3;
    tm = 16 * sq_r + 4 * (xcd & 3) + (j & 3);
    tn = 16 * sq_c + 8 * (xcd >> 2) + (j >> 2);
}


// LDS pointer types for the direct-to-LDS buffer loads and transposing reads.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding): vmcnt <= n, lgkmcnt = 0, expcnt unconstrained.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | (((n >> 4) & 3) << 14); }


// Rebase a workgroup of a K-split grid (gridDim.y > 1) onto its k range and
// its partial-product slot; see GemmParams::kchunk.  T is the operand type.
template <typename T>
__device__ __forceinline__ void apply_k_split(GemmParams &p) {
    if (p.kchunk <= 0) return;
    const int kb = (int)blockIdx.y * p.kchunk;
    // k runs along a row of an untransposed A and a transposed B, down the
    // columns otherwise.
    p.A = static_cast<const T *>(p.A) + (p.op_a == GEMM_OP_N ? (int64_t)kb : (int64_t)kb * p.lda);
    p.B = static_cast<const T *>(p.B) + (p.op_b == GEMM_OP_N ? (int64_t)kb * p.ldb : (int64_t)kb);
    p.K = min(p.K - kb, p.kchunk);
    p.C = p.partials + (int64_t)blockIdx.y * p.M * p.N;
    p.ldc = p.N;
    p.alpha = 1.0f;
    p.beta = 0.0f;
    p.bias = nullptr;          // the reduce applies the epilogue once
    p.act = 0;
    p.out_type = GEMM_OUT_F32;     // partials are fp32, into the workspace
    p.out = p.C;
    p.ldo = p.ldc;
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (a rational function of t = 1 / (1 + p|x|) times exp(-x^2); the
// formula's error is at most 1.5e-7), evaluated inline: the library erff is
// a function call, and a call inside an epilogue forces the accumulator
// registers out to scratch memory.
__device__ __forceinline__ float erf_inline(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));       // 1 ulp reciprocal
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    // exp(-x^2) = 2^(-x^2 * log2(e)); the hardware exp2 is accurate to 1 ulp.
    return copysignf(1.0f - poly * __builtin_amdgcn_exp2f(-ax * ax * 1.44269504088896341f), x);
}

// The fused epilogue's activations ("Tiled matrix multiplication",
// "Implementation notes": bias and activation are applied while the tile is
// still in registers).  ReLU keeps NaN; GELU is the erf form,
// x * Phi(x) = x * (1 + erf(x / sqrt(2))) / 2, evaluated as written.  They
// are types so that a kernel holding a large accumulator tile can branch once
// on the activation and run one small loop body per case: a per-element
// branch makes the fully unrolled epilogue too large to unroll, and a loop
// over the accumulators with a run-time index puts them in scratch memory.
struct ActNone {
    __device__ static float apply(float v) { return v; }
};
struct ActRelu {
    __device__ static float apply(float v) { return v < 0.0f ? 0.0f : v; }
};
struct ActGelu {
    __device__ static float apply(float v) { return 0.5f * v * (1.0f + erf_inline(v * 0.70710678118654752f)); }
};

template <typename F>
__device__ __forceinline__ void with_activation(int act, F &&f) {
    if (act == GEMM_ACT_GELU) f(ActGelu{});
    else if (act == GEMM_ACT_RELU) f(ActRelu{});
    else f(ActNone{});
}

// The fused epilogue on one output value already holding
// alpha * acc + beta * C0: add the column's bias, then the activation.
__device__ __forceinline__ float epilogue_value(float v, int64_t col, const float *bias, int act) {
    if (bias != nullptr) v += bias[col];
    if (act == GEMM_ACT_RELU) v = ActRelu::apply(v);
    else if (act == GEMM_ACT_GELU) v = ActGelu::apply(v);
    return v;
}

// ---- Output quantisation (GemmParams::out_type).
//
// bfloat16: gfx950's fp32 -> bf16 conversion instruction (what a plain
// conversion to __bf16 compiles to there), which rounds to nearest, ties to
// even, overflows to infinity and keeps NaN a NaN.  One instruction per value
// instead of the bit arithmetic of a software rounding: the tile epilogues
// convert hundreds of values in one unrolled pass, and every extra temporary
// there competes with the accumulators for registers.
__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// OCP E4M3: saturate to +-448 first (both comparisons are false for NaN,
// which passes through to the NaN code), then the hardware conversion,
// which rounds to nearest, ties to even.
__device__ __forceinline__ uint8_t to_e4m3(float x) {
    x = x > 448.0f ? 448.0f : (x < -448.0f ? -448.0f : x);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false) & 0xff);
}

template <int OUT> struct OutType { static constexpr int value = OUT; };
// Calls f with the output type as a compile-time constant, so an epilogue
// branches once per tile rather than once per element.
template <class F> __device__ __forceinline__ void with_output(int out, F &&f) {
    if (out == GEMM_OUT_BF16) f(OutType<GEMM_OUT_BF16>{});
    else if (out == GEMM_OUT_FP8) f(OutType<GEMM_OUT_FP8>{});
    else f(OutType<GEMM_OUT_F32>{});
}

// One finished value at (row, col) of the output.
template <int OUT>
__device__ __forceinline__ void store_out(const GemmParams &p, int64_t row, int64_t col, float v) {
    if constexpr (OUT == GEMM_OUT_F32)
        p.C[row * p.ldc + col] = v;
    else if constexpr (OUT == GEMM_OUT_BF16)
        static_cast<uint16_t *>(p.out)[row * p.ldo + col] = to_bf16(v * p.out_scale);
    else
        static_cast<uint8_t *>(p.out)[row * p.ldo + col] = to_e4m3(v * p.out_scale);
}
// The same with the type read at run time (per-element epilogues).
__device__ __forceinline__ void store_out_any(const GemmParams &p, int64_t row, int64_t col, float v) {
    if (p.out_type == GEMM_OUT_BF16) store_out<GEMM_OUT_BF16>(p, row, col, v);
    else if (p.out_type == GEMM_OUT_FP8) store_out<GEMM_OUT_FP8>(p, row, col, v);
    else store_out<GEMM_OUT_F32>(p, row, col, v);
}

// Register-staged kernels whose epilogue holds more than 128 accumulators per
// lane store fp32 only: a run-time output switch per element (even a
// rewritten fp32 store) pushes their accumulators to scratch.  Their table
// rows say so.
constexpr bool quantising_epilogue(int acc_per_lane) { return acc_per_lane <= 128; }

// Whether four output values of a row starting at a column that is a
// multiple of 4 form one aligned vector (16, 8 or 4 bytes).
template <int OUT> __device__ __forceinline__ bool out_vec4(const GemmParams &p) {
    if constexpr (OUT == GEMM_OUT_F32)
        return (reinterpret_cast<uintptr_t>(p.C) & 15) == 0 && p.ldc % 4 == 0;
    else
        return (reinterpret_cast<uintptr_t>(p.out) & (OUT == GEMM_OUT_BF16 ? 7 : 3)) == 0 && p.ldo % 4 == 0;
}

// The first n (1..3) of four values of a run cut by the edge of C.
template <int OUT>
__device__ __forceinline__ void store_out_first(const GemmParams &p, int64_t row, int64_t col, f32x4 v, int n) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
        if (t < n) store_out<OUT>(p, row, col + t, v[t]);
}

// Four finished values of row `row`, columns col .. col+3; `vec` as out_vec4.
template <int OUT>
__device__ __forceinline__ void store_out4(const GemmParams &p, int64_t row, int64_t col, f32x4 v, bool vec) {
    if constexpr (OUT == GEMM_OUT_F32) {
        float *cp = p.C + row * p.ldc + col;
        if (vec) {
            *reinterpret_cast<f32x4 *>(cp) = v;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) cp[t] = v[t];
        }
    } else if constexpr (OUT == GEMM_OUT_BF16) {
        const uint32_t h0 = to_bf16(v[0] * p.out_scale), h1 = to_bf16(v[1] * p.out_scale);
        const uint32_t h2 = to_bf16(v[2] * p.out_scale), h3 = to_bf16(v[3] * p.out_scale);
        uint16_t *op = static_cast<uint16_t *>(p.out) + row * p.ldo + col;
        if (vec) {
            *reinterpret_cast<u32x2 *>(op) = u32x2{h0 | (h1 << 16), h2 | (h3 << 16)};
        } else {
            op[0] = (uint16_t)h0;
            op[1] = (uint16_t)h1;
            op[2] = (uint16_t)h2;
            op[3] = (uint16_t)h3;
        }
    } else {
        const uint32_t b0 = to_e4m3(v[0] * p.out_scale), b1 = to_e4m3(v[1] * p.out_scale);
        const uint32_t b2 = to_e4m3(v[2] * p.out_scale), b3 = to_e4m3(v[3] * p.out_scale);
        uint8_t *op = static_cast<uint8_t *>(p.out) + row * p.ldo + col;
        if (vec) {
            *reinterpret_cast<uint32_t *>(op) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        } else {
            op[0] = (uint8_t)b0;
            op[1] = (uint8_t)b1;
            op[2] = (uint8_t)b2;
            op[3] = (uint8_t)b3;
        }
    }
}

}  // namespace gemm
