/*
 * abi_consumer.c -- a plain C program that uses libarrms.so through
 * include/arrms.h alone: device memory and a stream from the HIP runtime API,
 * no PyTorch and no Python. It runs the fused epilogue (the rank-ordered sum,
 * residual add and RMSNorm of the custom all-reduce pages, ROCm/aiter PR #6699
 * "gfx1250 fused all-reduce + RMSNorm", section Changes) on both paths and
 * checks every output byte against the CPU oracle (liboracle.so, test
 * infrastructure), then checks a few error returns. Prints "abi_consumer ok"
 * and exits 0 on success; any mismatch or failed call exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "arrms.h"

/* the CPU oracle (oracle/oracle.c) */
int oracle_fused_rows(const void *const *rank_in, int R, const void *residual, const void *weight, void *out,
                      void *residual_out, void *fp8_out, float *fp8_scale, int M, int H, float eps, int flags,
                      int row_begin, int row_end, float *h_scratch);
#define ORC_GEMMA 4
#define ORC_FP8 8

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform(void) /* xorshift64*, in [0, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t bf16_rne(float f) /* finite values: round to nearest, ties to even */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int compare(const char *what, const void *got, const void *want, size_t bytes)
{
    if (memcmp(got, want, bytes) == 0)
        return 0;
    size_t n = 0;
    for (size_t i = 0; i < bytes; ++i)
        n += ((const uint8_t *)got)[i] != ((const uint8_t *)want)[i];
    fprintf(stderr, "%s: %zu of %zu bytes differ\n", what, n, bytes);
    return 1;
}

/* One case: R bf16 rank inputs [M][H] ~ U(-scale, scale), residual U(-1, 1),
 * weight 1 + U(-0.1, 0.1) (or U(-0.1, 0.1) under gemma); FP8 output with the
 * T mirror when fp8 is set. Both paths, one stream. */
static int run_case(int R, int M, int H, int gemma, int fp8, float eps, hipStream_t st)
{
    const size_t n = (size_t)M * H, tb = n * 2;
    uint16_t *hx[ARRMS_MAX_RANKS], *hres = malloc(tb), *hw = malloc((size_t)H * 2);
    for (int r = 0; r < R; ++r) {
        hx[r] = malloc(tb);
        const double scale = 0.5 + 4.0 * r;
        for (size_t i = 0; i < n; ++i)
            hx[r][i] = bf16_rne((float)((2.0 * uniform() - 1.0) * scale));
    }
    for (size_t i = 0; i < n; ++i)
        hres[i] = bf16_rne((float)(2.0 * uniform() - 1.0));
    for (int j = 0; j < H; ++j)
        hw[j] = bf16_rne((float)((gemma ? 0.0 : 1.0) + 0.2 * uniform() - 0.1));

    /* the oracle's answer */
    uint16_t *wout = malloc(tb), *wrout = malloc(tb);
    uint8_t *wq = malloc(n);
    float *wsc = malloc((size_t)M * 4), *scratch = malloc((size_t)H * 4);
    const int oflags = (gemma ? ORC_GEMMA : 0) | (fp8 ? ORC_FP8 : 0);
    if (oracle_fused_rows((const void *const *)hx, R, hres, hw, wout, wrout, fp8 ? wq : NULL, fp8 ? wsc : NULL, M, H,
                          eps, oflags, 0, M, scratch) != 0) {
        fprintf(stderr, "oracle rejected the case\n");
        return 1;
    }

    /* device buffers */
    void *dx[ARRMS_MAX_RANKS], *dres, *dw, *dout, *drout, *dq = NULL, *dsc = NULL;
    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipMalloc(&dx[r], tb));
        CHECK_HIP(hipMemcpy(dx[r], hx[r], tb, hipMemcpyHostToDevice));
    }
    CHECK_HIP(hipMalloc(&dres, tb));
    CHECK_HIP(hipMalloc(&dw, (size_t)H * 2));
    CHECK_HIP(hipMalloc(&dout, tb));
    CHECK_HIP(hipMalloc(&drout, tb));
    CHECK_HIP(hipMemcpy(dres, hres, tb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dw, hw, (size_t)H * 2, hipMemcpyHostToDevice));
    if (fp8) {
        CHECK_HIP(hipMalloc(&dq, n));
        CHECK_HIP(hipMalloc(&dsc, (size_t)M * 4));
    }

    int bad = 0;
    uint16_t *gout = malloc(tb), *grout = malloc(tb);
    uint8_t *gq = malloc(n);
    float *gsc = malloc((size_t)M * 4);
    const int paths[2] = {ARRMS_FORCE_ONE_STAGE, ARRMS_FORCE_TWO_STAGE};
    for (int p = 0; p < 2; ++p) {
        const int flags = ARRMS_DTYPE_BF16 | (gemma ? ARRMS_GEMMA : 0) | (fp8 ? ARRMS_FP8 : 0) | paths[p];
        CHECK_HIP(hipMemsetAsync(dout, 0xff, tb, st));
        CHECK_HIP(hipMemsetAsync(drout, 0xff, tb, st));
        const int rc = arrms_fused((const void *const *)dx, R, dres, dw, dout, drout, dq, (float *)dsc, M, H, eps,
                                   flags, st);
        if (rc != ARRMS_OK) {
            fprintf(stderr, "arrms_fused: %s\n", arrms_status_string(rc));
            return 1;
        }
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_HIP(hipMemcpy(gout, dout, tb, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(grout, drout, tb, hipMemcpyDeviceToHost));
        bad |= compare("residual_out", grout, wrout, tb);
        bad |= compare("out", gout, wout, tb);
        if (fp8) {
            CHECK_HIP(hipMemcpy(gq, dq, n, hipMemcpyDeviceToHost));
            CHECK_HIP(hipMemcpy(gsc, dsc, (size_t)M * 4, hipMemcpyDeviceToHost));
            bad |= compare("fp8 codes", gq, wq, n);
            bad |= compare("fp8 scales", gsc, wsc, (size_t)M * 4);
        }
        printf("case R=%d M=%d H=%d bf16%s%s path=%s: %s\n", R, M, H, gemma ? " gemma" : "", fp8 ? " fp8" : "",
               p ? "two" : "one", bad ? "MISMATCH" : "bit-identical to the oracle");
    }

    /* error returns: nothing is launched or written */
    const int mis = arrms_fused((const void *const *)dx, R, (const char *)dres + 2, dw, dout, drout, dq,
                                (float *)dsc, M, H, eps, ARRMS_DTYPE_BF16 | (fp8 ? ARRMS_FP8 : 0), st);
    const int both = arrms_fused((const void *const *)dx, R, dres, dw, dout, drout, dq, (float *)dsc, M, H, eps,
                                 ARRMS_FORCE_ONE_STAGE | ARRMS_FORCE_TWO_STAGE | (fp8 ? ARRMS_FP8 : 0), st);
    if (mis != ARRMS_ERR_UNSUPPORTED || both != ARRMS_ERR_INVALID || !arrms_status_string(mis)) {
        fprintf(stderr, "error returns: misaligned %d, two forced paths %d\n", mis, both);
        bad = 1;
    }

    for (int r = 0; r < R; ++r) {
        CHECK_HIP(hipFree(dx[r]));
        free(hx[r]);
    }
    CHECK_HIP(hipFree(dres));
    CHECK_HIP(hipFree(dw));
    CHECK_HIP(hipFree(dout));
    CHECK_HIP(hipFree(drout));
    if (fp8) {
        CHECK_HIP(hipFree(dq));
        CHECK_HIP(hipFree(dsc));
    }
    free(hres); free(hw); free(wout); free(wrout); free(wq); free(wsc); free(scratch);
    free(gout); free(grout); free(gq); free(gsc);
    return bad;
}

int main(void)
{
    int count = 0;
    CHECK_HIP(hipGetDeviceCount(&count));
    if (count < 1) {
        fprintf(stderr, "no GPU\n");
        return 1;
    }
    CHECK_HIP(hipSetDevice(0));
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    if (arrms_query_path(1024, 6144, 4, ARRMS_DTYPE_BF16) != ARRMS_PATH_ONE_STAGE ||
        arrms_query_path(0, 6144, 4, ARRMS_DTYPE_BF16) != ARRMS_PATH_NONE) {
        fprintf(stderr, "arrms_query_path\n");
        return 1;
    }
    int bad = 0;
    bad |= run_case(4, 37, 6144, 0, 0, 1e-6f, st);
    bad |= run_case(3, 20, 2880, 1, 1, 1e-6f, st);
    bad |= run_case(8, 5, 7168, 0, 1, 1e-5f, st);
    CHECK_HIP(hipStreamDestroy(st));
    if (arrms_release_staging() != ARRMS_OK)
        bad = 1;
    if (bad) {
        fprintf(stderr, "abi_consumer FAILED\n");
        return 1;
    }
    printf("abi_consumer ok\n");
    return 0;
}
