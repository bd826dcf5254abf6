/*
 * Plain C99 client of libgemm: include/gemm.h must compile as C with strict
 * warnings, and the host-only entry points must behave as documented when
 * called from C (no GPU is touched: validation, planning, kernel queries and
 * workspace sizing run on the host).  Built and run by tests/test_c_abi.py.
 * Prints "OK <checks>" on success, "FAIL <what>" otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemm.h"

static int checks = 0;
#define CHECK(cond, what)                      \
    do {                                       \
        ++checks;                              \
        if (!(cond)) {                         \
            printf("FAIL %s\n", what);         \
            return 1;                          \
        }                                      \
    } while (0)

int main(void)
{
    /* Well-aligned stand-in device addresses: planning only inspects them. */
    const void *A = (const void *)(uintptr_t)0x7f0000000000ull;
    const void *B = (const void *)(uintptr_t)0x7f1000000000ull;
    float *C = (float *)(uintptr_t)0x7f2000000000ull;
    gemm_plan plan;
    gemm_kernel_info info;
    int32_t id, n = gemm_kernel_count();

    CHECK(n > 0, "kernel count");
    for (id = 1; id <= n; ++id) {
        CHECK(gemm_kernel_query(id, &info) == GEMM_OK, "kernel query");
        CHECK(info.id == id && info.name != NULL && strlen(info.name) > 0, "kernel info");
        CHECK(info.layouts >= 1 && info.layouts <= 15, "kernel layouts");
        CHECK((info.outputs & 1) && info.outputs <= 7, "kernel outputs (fp32 always)");
    }
    CHECK(gemm_kernel_query(0, &info) == GEMM_ERR_INVALID_ARG, "kernel id 0 rejected");

    CHECK(gemm_plan_query(GEMM_DTYPE_F32, 4096, 4096, 4096, 1.0f, A, 4096, B, 4096, 0.0f, C, 4096, 0, 0,
                          &plan) == GEMM_OK, "fp32 plan");
    CHECK(plan.path == GEMM_PATH_TILED && plan.tile_m == 256 && plan.grid == 256, "fp32 4096 plan shape");
    CHECK(gemm_plan_query(GEMM_DTYPE_F32, 16, 8192, 8192, 1.0f, A, 8192, B, 8192, 0.0f, C, 8192, 0, 0,
                          &plan) == GEMM_OK && plan.path == GEMM_PATH_SKINNY, "skinny plan");
    CHECK(gemm_plan_query_general(GEMM_DTYPE_FP8F32, GEMM_OP_N, GEMM_OP_T, 8192, 8192, 8192, 1.0f, A, 8192, B,
                                  8192, 0.0f, C, 8192, 0, 0, &plan) == GEMM_OK, "fp8 plan");
    CHECK(gemm_kernel_query(plan.kernel_id, &info) == GEMM_OK && info.dtype == GEMM_DTYPE_FP8F32 &&
          info.layouts == 2, "fp8 B-transposed kernel");

    /* Errors come back before any device call. */
    CHECK(gemm_f32(-1, 4, 4, 1.0f, (const float *)A, 4, (const float *)B, 4, 0.0f, C, 4, NULL) ==
          GEMM_ERR_INVALID_ARG, "negative M");
    CHECK(gemm_general(9, GEMM_OP_N, GEMM_OP_N, 4, 4, 4, 1.0f, A, 4, B, 4, 0.0f, C, 4, 0, NULL, NULL, 0, NULL) ==
          GEMM_ERR_INVALID_ARG, "unknown dtype");
    {
        gemm_epilogue epi;
        memset(&epi, 0, sizeof epi);
        epi.activation = 7;
        CHECK(gemm_f32_epi(4, 4, 4, 1.0f, (const float *)A, 4, (const float *)B, 4, 0.0f, C, 4, &epi, NULL, 0,
                           NULL) == GEMM_ERR_INVALID_ARG, "unknown activation");
        epi.activation = GEMM_ACT_GELU;
        CHECK(gemm_bf16f32_epi(0, 4, 4, 1.0f, (const uint16_t *)A, 4, (const uint16_t *)B, 4, 0.0f, C, 4, &epi,
                               NULL, 0, NULL) == GEMM_OK, "empty call is a no-op");
        /* Quantised output: the plan takes a kernel that writes it; a NULL
         * output, an unknown type or ldo < N is rejected. */
        epi.activation = GEMM_ACT_NONE;
        epi.out_type = GEMM_OUT_BF16;
        epi.out = (void *)(uintptr_t)0x7f3000000000ull;
        epi.ldo = 4096;
        CHECK(gemm_plan_query_epi(GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_N, 4096, 4096, 4096, 1.0f, A, 4096, B, 4096,
                                  0.0f, NULL, 4096, 0, &epi, 0, &plan) == GEMM_OK, "bf16-output plan, C NULL");
        CHECK(gemm_kernel_query(plan.kernel_id, &info) == GEMM_OK && (info.outputs & (1 << GEMM_OUT_BF16)),
              "bf16-output kernel");
        epi.ldo = 4095;
        CHECK(gemm_plan_query_epi(GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_N, 4096, 4096, 4096, 1.0f, A, 4096, B, 4096,
                                  0.0f, NULL, 4096, 0, &epi, 0, &plan) == GEMM_ERR_INVALID_ARG, "ldo < N");
        epi.ldo = 4096;
        epi.out = NULL;
        CHECK(gemm_f32_epi(4, 4, 4, 1.0f, (const float *)A, 4, (const float *)B, 4, 0.0f, C, 4, &epi, NULL, 0,
                           NULL) == GEMM_ERR_INVALID_ARG, "NULL output");
        epi.out_type = 3;
        CHECK(gemm_f32_epi(4, 4, 4, 1.0f, (const float *)A, 4, (const float *)B, 4, 0.0f, C, 4, &epi, NULL, 0,
                           NULL) == GEMM_ERR_INVALID_ARG, "unknown output type");
    }
    CHECK(gemm_workspace_size(GEMM_DTYPE_BF16F32, 256, 512, 6000) > 0, "workspace size");
    CHECK(gemm_workspace_size(GEMM_DTYPE_F32, 4096, 4096, 4096) == 0, "no workspace for a full wave");
    CHECK(strcmp(gemm_status_string(GEMM_OK), "success") == 0, "status string");
    /* The no-allocation entry point checks its arguments, then the scratch
     * its K split could need, before touching the device. */
    CHECK(gemm_general_noalloc(GEMM_DTYPE_F32, GEMM_OP_N, GEMM_OP_N, -1, 4, 4, 1.0f, A, 4, B, 4, 0.0f, C, 4, 0,
                               NULL, NULL) == GEMM_ERR_INVALID_ARG, "noalloc invalid size");
    CHECK(gemm_general_noalloc(GEMM_DTYPE_BF16F32, GEMM_OP_N, GEMM_OP_N, 2048, 2048, 65536, 1.0f, A, 65536, B, 2048,
                               0.0f, C, 2048, 0, NULL, NULL) == GEMM_ERR_SCRATCH, "noalloc scratch limit");
    CHECK(GEMM_STATIC_SCRATCH_BYTES == ((int64_t)32 << 20), "scratch size macro");
    CHECK(gemm_tuning_count() >= 0, "tuning count");
    {
        gemm_plan pl;
        CHECK(gemm_autotune_general(GEMM_DTYPE_FP8F32, GEMM_OP_N, GEMM_OP_T, 64, 64, 64, 1.0f, A, 64, B, 64, 0.0f, C,
                                    64, NULL, 0, 0, NULL, &pl) == GEMM_ERR_INVALID_ARG, "autotune reps 0");
        CHECK(gemm_autotune_general(GEMM_DTYPE_FP8F32, GEMM_OP_N, 2, 64, 64, 64, 1.0f, A, 64, B, 64, 0.0f, C, 64,
                                    NULL, 0, 5, NULL, &pl) == GEMM_ERR_INVALID_ARG, "autotune bad op");
    }

    printf("OK %d\n", checks);
    return 0;
}
