/*
 * A plain C program that uses libmoe_finalize.so through include/moe_finalize.h
 * alone: HIP runtime calls for memory and a stream, no Python, no torch.
 * tests/test_gpu_c_driver.py writes the inputs, runs this program and
 * compares what it wrote with the oracle.
 *
 *   capi_c_driver DIR T H K R S WDT EPS GAIN_CENTER WBN  CAP BK BH LIVE SCALE
 *
 * DIR holds the inputs as raw little-endian arrays:
 *   gemm2.bin [R, S] bf16, weights.bin [T, K] (WDT 1 = bf16, 2 = f32),
 *   idx.bin [T, K] int32, norm_weight.bin [H] bf16,
 *   beam_rows.bin [CAP, BK, BH] bf16, beam_weights.bin [CAP, BK] f32.
 * It writes out_rmsnorm.bin and out_finalize.bin [T, H] bf16 and out_beam.bin
 * [LIVE, BH] bf16 (token-major finalize, no norm, routed_scale SCALE), and
 * checks on the way that invalid calls return their status code and leave
 * the output untouched.  Exit status 0 when all went as expected; every
 * failure is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_finalize.h"

static int failures = 0;

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call,          \
                    hipGetErrorString(e_));                                       \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

static void expect(int cond, const char *what) {
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        failures++;
    }
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        perror(path);
        exit(2);
    }
    void *buf = malloc(bytes ? bytes : 1);
    size_t got = fread(buf, 1, bytes, f);
    fclose(f);
    if (got != bytes) {
        fprintf(stderr, "%s: expected %zu bytes, read %zu\n", path, bytes, got);
        exit(2);
    }
    return buf;
}

static void write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(buf, 1, bytes, f) != bytes) {
        perror(path);
        exit(2);
    }
    fclose(f);
}

/* Device copy of `bytes` bytes of `host`, or an uninitialised buffer when host is NULL. */
static void *to_device(const void *host, size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (host && bytes)
        HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* Reads the device buffer back and reports whether every byte still holds `fill`. */
static int untouched(const void *dev, size_t bytes, unsigned char fill) {
    unsigned char *h = (unsigned char *)malloc(bytes);
    HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    int ok = 1;
    for (size_t i = 0; i < bytes; i++)
        ok &= h[i] == fill;
    free(h);
    return ok;
}

static void expect_status(int got, int want, const char *what) {
    char msg[256];
    snprintf(msg, sizeof msg, "%s: status %d (%s), expected %d", what, got,
             mf_status_string(got), want);
    expect(got == want, msg);
    expect(mf_status_string(got)[0] != '\0', "every status has a description");
    if (got != MF_ERR_LAUNCH_FAILED)
        expect(mf_last_error_message()[0] == '\0', "no launch error is recorded");
}

int main(int argc, char **argv) {
    if (argc != 16) {
        fprintf(stderr, "usage: %s DIR T H K R S WDT EPS GAIN_CENTER WBN CAP BK BH LIVE SCALE\n",
                argv[0]);
        return 2;
    }
    const char *dir = argv[1];
    const int64_t T = atoll(argv[2]);
    const int32_t H = atoi(argv[3]), K = atoi(argv[4]);
    const int64_t R = atoll(argv[5]), S = atoll(argv[6]);
    const int32_t wdt = atoi(argv[7]);
    const float eps = strtof(argv[8], NULL), gain_center = strtof(argv[9], NULL);
    const int32_t wbn = atoi(argv[10]);
    const int64_t cap = atoll(argv[11]);
    const int32_t bk = atoi(argv[12]), bh = atoi(argv[13]);
    const int64_t live = atoll(argv[14]);
    const float scale = strtof(argv[15], NULL);
    const size_t wbytes = wdt == MF_DTYPE_BF16 ? 2 : 4;

    void *h_rows = read_file(dir, "gemm2.bin", (size_t)(R * S * 2));
    void *h_w = read_file(dir, "weights.bin", (size_t)(T * K) * wbytes);
    void *h_idx = read_file(dir, "idx.bin", (size_t)(T * K) * 4);
    void *h_nw = read_file(dir, "norm_weight.bin", (size_t)H * 2);
    void *h_brows = read_file(dir, "beam_rows.bin", (size_t)(cap * bk * bh) * 2);
    void *h_bw = read_file(dir, "beam_weights.bin", (size_t)(cap * bk) * 4);

    void *rows = to_device(h_rows, (size_t)(R * S * 2));
    void *w = to_device(h_w, (size_t)(T * K) * wbytes);
    int32_t *idx = (int32_t *)to_device(h_idx, (size_t)(T * K) * 4);
    void *nw = to_device(h_nw, (size_t)H * 2);
    void *brows = to_device(h_brows, (size_t)(cap * bk * bh) * 2);
    float *bw = (float *)to_device(h_bw, (size_t)(cap * bk) * 4);
    const size_t out_bytes = (size_t)(T * H) * 2, bout_bytes = (size_t)(live * bh) * 2;
    void *out_n = to_device(NULL, out_bytes), *out_f = to_device(NULL, out_bytes);
    void *bout = to_device(NULL, bout_bytes);
    HIP_OK(hipMemset(out_n, 0xA5, out_bytes));
    HIP_OK(hipMemset(out_f, 0xA5, out_bytes));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* invalid calls first: each returns its code and leaves out_n untouched */
    expect_status(moe_finalize_rmsnorm(rows, R, S, w, wdt, idx, nw, out_n, T, 100, K, eps,
                                       gain_center, wbn, stream),
                  MF_ERR_BAD_SHAPE, "hidden 100");
    expect_status(moe_finalize_rmsnorm(rows, R, S, w, wdt, idx, nw, NULL, T, H, K, eps,
                                       gain_center, wbn, stream),
                  MF_ERR_NULL_POINTER, "NULL output");
    expect_status(moe_finalize_rmsnorm(rows, R, S, w, wdt, idx, nw, (char *)out_n + 2, T, H, K,
                                       eps, gain_center, wbn, stream),
                  MF_ERR_MISALIGNED, "output off by one element");
    expect_status(moe_finalize_rmsnorm(rows, R, S, w, 7, idx, nw, out_n, T, H, K, eps,
                                       gain_center, wbn, stream),
                  MF_ERR_BAD_DTYPE, "weights dtype 7");
    expect_status(moe_finalize(rows, R, S + 4, w, wdt, idx, out_n, T, H, K, stream),
                  MF_ERR_MISALIGNED, "row stride not a multiple of 8");
    expect_status(beam_moe_finalize(brows, cap, bk, bh, bw, cap, bout, cap + 1, NULL, scale, 0.0f,
                                    0, stream),
                  MF_ERR_BAD_SHAPE, "live tokens above capacity");
    HIP_OK(hipStreamSynchronize(stream));
    expect(untouched(out_n, out_bytes, 0xA5), "output untouched by invalid calls");

    /* the three computations, all on the caller's stream */
    expect_status(moe_finalize_rmsnorm(rows, R, S, w, wdt, idx, nw, out_n, T, H, K, eps,
                                       gain_center, wbn, stream),
                  MF_OK, "moe_finalize_rmsnorm");
    expect_status(moe_finalize(rows, R, S, w, wdt, idx, out_f, T, H, K, stream), MF_OK,
                  "moe_finalize");
    expect_status(beam_moe_finalize(brows, cap, bk, bh, bw, cap, bout, live, NULL, scale, 0.0f, 0,
                                    stream),
                  MF_OK, "beam_moe_finalize");
    HIP_OK(hipStreamSynchronize(stream));

    void *h_out = malloc(out_bytes > bout_bytes ? out_bytes : bout_bytes);
    HIP_OK(hipMemcpy(h_out, out_n, out_bytes, hipMemcpyDeviceToHost));
    write_file(dir, "out_rmsnorm.bin", h_out, out_bytes);
    HIP_OK(hipMemcpy(h_out, out_f, out_bytes, hipMemcpyDeviceToHost));
    write_file(dir, "out_finalize.bin", h_out, out_bytes);
    HIP_OK(hipMemcpy(h_out, bout, bout_bytes, hipMemcpyDeviceToHost));
    write_file(dir, "out_beam.bin", h_out, bout_bytes);

    HIP_OK(hipStreamDestroy(stream));
    void *bufs[] = {rows, w, idx, nw, brows, bw, out_n, out_f, bout};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++)
        HIP_OK(hipFree(bufs[i]));
    void *hbufs[] = {h_rows, h_w, h_idx, h_nw, h_brows, h_bw, h_out};
    for (size_t i = 0; i < sizeof hbufs / sizeof hbufs[0]; i++)
        free(hbufs[i]);
    printf("capi_c_driver: %s\n", failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
