// Epilogue shared by the whole-line kernels (gemm_bf16_lines.hip,
// gemm_fp8_lines.hip): each wave's accumulators pass through LDS so that every
// store instruction writes four rows of 256 contiguous bytes (the coalescing
// rung of "A GEMM Kernel, Step by Step", taken to the cache line).
#pragma once

#include "gemm_device.hpp"

namespace gemm {

// The epilogue runs in passes of 64 columns per wave (FN / 2 of them for a
// wave tile of FM x FN fragments of 32 x 32).  The wave's 32*FM x 64
// accumulators of a pass are written to its LDS (stage_row(r) points at row
// r, 256 bytes) in their register layout (register 4g + t of lane (h, l32)
// in fragment (fm, fn) is row 32fm + l32, column 32*(fn%2) + 8g + 4h + t of
// the pass; 16-byte chunk c of a row at c ^ (row & 15), for both the
// accumulator-layout writes and the row-major reads), then read back 4 rows
// x 64 columns per instruction and finished and stored a row run at a time.
// STRADDLE: N is free, and runs of 4 columns that straddle it are read and
// stored element by element (otherwise N is a multiple of 8).
template <int OUT, bool STRADDLE, typename RowPtr, int FM = 4, int FN = 4>
__device__ __forceinline__ void lines_epilogue(const GemmParams &p, const f32x16 (&acc)[FM][FN], RowPtr stage_row,
                                               int m0, int n0, int wm, int wn, int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int M = p.M, N = p.N;
    const float alpha = p.alpha, beta = p.beta;
    const bool vec_c = ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0) && (p.ldc % 4 == 0);
    const bool vec_o = out_vec4<OUT>(p);
    const int act = p.act;
#pragma unroll
    for (int pass = 0; pass < FN / 2; ++pass) {
#pragma unroll
        for (int fl = 0; fl < 2; ++fl) {
            const int fn = 2 * pass + fl;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = 32 * fm + l32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = (8 * fl + 2 * g + h) ^ (row & 15);
                    const f32x4 v = {acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
                                     acc[fm][fn][4 * g + 3]};
                    *reinterpret_cast<f32x4 *>(stage_row(row) + 16 * c) = v;
                }
            }
        }
        const int cc = lane & 15;
        const int col = n0 + wn * 32 * FN + 64 * pass + 4 * cc;
        float b[4];   // -0.0 is the identity of IEEE addition, signed zeros included
#pragma unroll
        for (int t = 0; t < 4; ++t)
            b[t] = (p.bias != nullptr && (STRADDLE ? col + t < N : col < N)) ? p.bias[col + t] : -0.0f;
        const bool whole = !STRADDLE || col + 4 <= N;
        // C = A x B (alpha 1, beta 0, no bias or activation): each run is
        // stored as read, and eight runs are read from LDS before any is
        // stored (3% of the whole 8192^3 call against the general loop
        // below, whose per-run steps and uniform branches the compiler
        // keeps in order).
        if (alpha == 1.0f && beta == 0.0f && p.bias == nullptr && act == GEMM_ACT_NONE) {
            for (int i0 = 0; i0 < 8 * FM; i0 += 8) {
                f32x4 vv[8];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const int row = 4 * (i0 + ii) + (lane >> 4);
                    vv[ii] = *reinterpret_cast<const f32x4 *>(stage_row(row) + 16 * (cc ^ (row & 15)));
                }
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const int grow = m0 + wm * 32 * FM + 4 * (i0 + ii) + (lane >> 4);
                    if (grow >= M || col >= N) continue;
                    if (whole)
                        store_out4<OUT>(p, grow, col, vv[ii], vec_o);
                    else
                        store_out_first<OUT>(p, grow, col, vv[ii], N - col);
                }
            }
            continue;
        }
#pragma unroll 4
        for (int i = 0; i < 8 * FM; ++i) {
            const int row = 4 * i + (lane >> 4);
            f32x4 v = *reinterpret_cast<const f32x4 *>(stage_row(row) + 16 * (cc ^ (row & 15)));
            const int grow = m0 + wm * 32 * FM + row;
            if (grow >= M || col >= N) continue;
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] *= alpha;
            if (beta != 0.0f) {
                const float *cp = p.C + (int64_t)grow * p.ldc + col;
                f32x4 c0;
                if (whole && vec_c) {
                    c0 = *reinterpret_cast<const f32x4 *>(cp);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) c0[t] = (!STRADDLE || col + t < N) ? cp[t] : 0.0f;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = fmaf(beta, c0[t], v[t]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] += b[t];
            if (act == GEMM_ACT_GELU) {
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = ActGelu::apply(v[t]);
            } else if (act == GEMM_ACT_RELU) {
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = ActRelu::apply(v[t]);
            }
            if (whole)
                store_out4<OUT>(p, grow, col, v, vec_o);
            else
                store_out_first<OUT>(p, grow, col, v, N - col);
        }
    }
}

}  // namespace gemm
