/* The front through libqkvfront from a C program that uses no PyTorch:
 * device memory, a stream and copies come from the HIP runtime's C API.
 * It reads one call's inputs from DIR (raw little-endian arrays written by
 * the test), checks the call with qkvf_check, runs qkvf_prepare and then
 * qkvf_run twice on its own stream, requires both calls to give the same y
 * bits and no call to have given up, and writes y and the cache back to DIR
 * for the test to compare with the oracle.
 *
 * usage: gpu_front DIR N NUM_KV_HEADS M TABLE_ROWS PAGES
 *   DIR/x.bin        bf16 [M][8192]
 *   DIR/W.bin        bf16 [N][8192]
 *   DIR/positions.bin, DIR/slots.bin   int64 [M]
 *   DIR/cos_sin.bin  fp32 [TABLE_ROWS][64]
 *   DIR/cache.bin    bf16 [PAGES][NUM_KV_HEADS][16][128]
 * writes DIR/y.bin (bf16 [M][N]) and DIR/cache_out.bin. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qkvf.h"

#define HIP_TRY(call)                                                                 \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

#define QKVF_TRY(call)                                                                \
    do {                                                                              \
        int s_ = (call);                                                              \
        if (s_ != QKVF_OK) {                                                          \
            fprintf(stderr, "%s failed: %s\n", #call, qkvf_strerror(s_));             \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static void *slurp(const char *dir, const char *name, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    void *buf = malloc(bytes);
    int ok = f != NULL && buf != NULL && fread(buf, 1, bytes, f) == bytes;
    if (f != NULL)
        ok = ok && fgetc(f) == EOF;   /* the file holds exactly `bytes` */
    if (f != NULL)
        fclose(f);
    if (!ok) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
        free(buf);
        return NULL;
    }
    return buf;
}

static int spill(const char *dir, const char *name, const void *buf, size_t bytes)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    int ok = f != NULL && fwrite(buf, 1, bytes, f) == bytes;
    if (f != NULL)
        ok = fclose(f) == 0 && ok;
    if (!ok)
        fprintf(stderr, "cannot write %s\n", path);
    return ok ? 0 : 1;
}

int main(int argc, char **argv)
{
    if (argc != 7) {
        fprintf(stderr, "usage: %s DIR N NUM_KV_HEADS M TABLE_ROWS PAGES\n", argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    const int N = atoi(argv[2]), nkv = atoi(argv[3]), M = atoi(argv[4]);
    const int64_t rows = atoll(argv[5]), pages = atoll(argv[6]);
    /* Shape and rows first, so the sizes below are those of a valid call. */
    QKVF_TRY(qkvf_plan(N, M, NULL, NULL, NULL, NULL));
    if (rows <= 0 || pages <= 0) {
        fprintf(stderr, "TABLE_ROWS and PAGES must be positive\n");
        return 2;
    }
    const size_t bx = (size_t)M * 8192 * 2, bw = (size_t)N * 8192 * 2, bi = (size_t)M * 8;
    const size_t bcs = (size_t)rows * 64 * 4, by = (size_t)M * N * 2;
    const size_t bc = (size_t)pages * nkv * 16 * 128 * 2;

    void *hx = slurp(dir, "x.bin", bx), *hw = slurp(dir, "W.bin", bw);
    void *hp = slurp(dir, "positions.bin", bi), *hs = slurp(dir, "slots.bin", bi);
    void *hcs = slurp(dir, "cos_sin.bin", bcs), *hc = slurp(dir, "cache.bin", bc);
    void *hy[2] = {malloc(by), malloc(by)};
    if (!hx || !hw || !hp || !hs || !hcs || !hc || !hy[0] || !hy[1])
        return 1;

    void *dx, *dw, *dp, *ds, *dcs, *dy, *dc;
    HIP_TRY(hipMalloc(&dx, bx));
    HIP_TRY(hipMalloc(&dw, bw));
    HIP_TRY(hipMalloc(&dp, bi));
    HIP_TRY(hipMalloc(&ds, bi));
    HIP_TRY(hipMalloc(&dcs, bcs));
    HIP_TRY(hipMalloc(&dy, by));
    HIP_TRY(hipMalloc(&dc, bc));
    HIP_TRY(hipMemcpy(dx, hx, bx, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(dw, hw, bw, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(dp, hp, bi, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(ds, hs, bi, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(dcs, hcs, bcs, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(dc, hc, bc, hipMemcpyHostToDevice));

    /* The full check reads the positions and slots back (it synchronizes). */
    QKVF_TRY(qkvf_check(N, nkv, M, pages, rows, dx, dw, (const int64_t *)dp,
                        (const int64_t *)ds, (const float *)dcs, dy, dc, 1));
    QKVF_TRY(qkvf_prepare(N, nkv, M));
    hipStream_t stream;
    HIP_TRY(hipStreamCreate(&stream));
    for (int call = 0; call < 2; ++call) {
        HIP_TRY(hipMemset(dy, 0x7F, by));   /* every y word a NaN canary */
        QKVF_TRY(qkvf_run(dx, dw, (const int64_t *)dp, (const int64_t *)ds,
                          (const float *)dcs, dy, dc, M, stream));
        HIP_TRY(hipStreamSynchronize(stream));
        HIP_TRY(hipMemcpy(hy[call], dy, by, hipMemcpyDeviceToHost));
    }
    QKVF_TRY(qkvf_device_fault());
    if (memcmp(hy[0], hy[1], by) != 0) {
        fprintf(stderr, "two calls gave different y bits\n");
        return 1;
    }
    HIP_TRY(hipMemcpy(hc, dc, bc, hipMemcpyDeviceToHost));
    if (spill(dir, "y.bin", hy[0], by) || spill(dir, "cache_out.bin", hc, bc))
        return 1;

    qkvf_release();
    HIP_TRY(hipStreamDestroy(stream));
    void *dev[] = {dx, dw, dp, ds, dcs, dy, dc};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
        HIP_TRY(hipFree(dev[i]));
    void *host[] = {hx, hw, hp, hs, hcs, hc, hy[0], hy[1]};
    for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i)
        free(host[i]);
    printf("ok: M=%d N=%d nkv=%d, two calls bitwise equal\n", M, N, nkv);
    return 0;
}
