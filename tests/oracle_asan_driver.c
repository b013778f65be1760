/*
 * Drives every CPU-oracle entry point on small inputs, including the edge
 * cases (invalid indices of every kind, no rows at all, zero tokens, padded
 * strides, NULL optional weights), so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check the oracle's memory accesses.
 * Test infrastructure (see tests/test_oracle_sanitized.py).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_round_to_bf16(double x);
int oracle_routed_sum(const uint16_t *, int64_t, int64_t, const void *, int32_t,
                      const int32_t *, float *, int64_t, int32_t, int32_t);
int oracle_moe_finalize(const uint16_t *, int64_t, int64_t, const void *, int32_t,
                        const int32_t *, uint16_t *, int64_t, int32_t, int32_t);
int oracle_moe_finalize_rmsnorm(const uint16_t *, int64_t, int64_t, const void *, int32_t,
                                const int32_t *, const uint16_t *, uint16_t *, int64_t,
                                int32_t, int32_t, float, float, int32_t);
int oracle_rmsnorm(const uint16_t *, int64_t, const uint16_t *, uint16_t *, int64_t,
                   int32_t, float, float, int32_t);
int oracle_beam_moe_finalize(const uint16_t *, int64_t, int32_t, int32_t, const float *,
                             uint16_t *, int64_t, const uint16_t *, float, float, int32_t);
int oracle_beam_norm_residual_norm(const uint16_t *, int64_t, const uint16_t *,
                                   const uint16_t *, const uint16_t *, uint16_t *, uint16_t *,
                                   int64_t, int32_t, float, float, float, float, int32_t,
                                   int32_t);
int oracle_beam_moe_finalize_norm_residual_norm(const uint16_t *, int64_t, int32_t, int32_t,
                                                const float *, const uint16_t *,
                                                const uint16_t *, const uint16_t *,
                                                uint16_t *, uint16_t *, int64_t, float, float,
                                                float, float, float, int32_t, int32_t);

static uint32_t state = 12345u;
static uint16_t rnd_bf16(void)
{
    state = state * 1664525u + 1013904223u;
    return (uint16_t)(0x3C00u + ((state >> 16) & 0x03FFu)) ^ (uint16_t)((state & 1u) << 15);
}

#define CHECK(x) do { if ((x) != 0) { fprintf(stderr, "failed: %s\n", #x); return 1; } } while (0)

int main(void)
{
    enum { H = 256, S = 264, R = 10, T = 5, K = 4 };
    /* exact-size heap allocations so that any overrun is caught */
    uint16_t *rows = malloc(sizeof(uint16_t) * R * S);
    float *w = malloc(sizeof(float) * T * K);
    uint16_t *wb = malloc(sizeof(uint16_t) * T * K);
    int32_t *idx = malloc(sizeof(int32_t) * T * K);
    uint16_t *nw = malloc(sizeof(uint16_t) * H);
    uint16_t *out = malloc(sizeof(uint16_t) * T * H);
    uint16_t *out2 = malloc(sizeof(uint16_t) * T * H);
    float *acc = malloc(sizeof(float) * T * H);
    uint16_t *e = malloc(sizeof(uint16_t) * T * K * H);
    uint16_t *res = malloc(sizeof(uint16_t) * T * H);
    for (int i = 0; i < R * S; ++i) rows[i] = rnd_bf16();
    for (int i = 0; i < T * K * H; ++i) e[i] = rnd_bf16();
    for (int i = 0; i < T * H; ++i) res[i] = rnd_bf16();
    for (int i = 0; i < H; ++i) nw[i] = rnd_bf16();
    const int32_t bad[] = {-1, INT32_MIN, R, R + 1, INT32_MAX};
    for (int i = 0; i < T * K; ++i) {
        idx[i] = (i % 3 == 0) ? bad[i % 5] : (int32_t)(i % R);
        w[i] = 0.25f;
        wb[i] = 0x3E80;
    }
    CHECK(oracle_routed_sum(rows, R, S, w, 1, idx, acc, T, H, K));
    CHECK(oracle_routed_sum(rows, R, S, wb, 0, idx, acc, T, H, K));
    CHECK(oracle_moe_finalize(rows, R, S, w, 1, idx, out, T, H, K));
    CHECK(oracle_moe_finalize(NULL, 0, S, w, 1, idx, out, T, H, K));   /* no rows */
    CHECK(oracle_moe_finalize(rows, R, S, w, 1, idx, out, 0, H, K));   /* no tokens */
    for (int wbn = 0; wbn < 2; ++wbn)
        CHECK(oracle_moe_finalize_rmsnorm(rows, R, S, w, 1, idx, nw, out, T, H, K, 1e-6f,
                                          1.0f, wbn));
    CHECK(oracle_rmsnorm(rows, S, nw, out, T, H, 1e-6f, 0.5f, 1));
    CHECK(oracle_beam_moe_finalize(e, T, K, H, w, out, T, NULL, 2.5f, 0.0f, 0));
    CHECK(oracle_beam_moe_finalize(e, T, K, H, w, out, T - 2, nw, 1.0f, 1e-6f, 1));
    CHECK(oracle_beam_moe_finalize(e, T, K, H, w, out, T, NULL, 1.0f, 1e-6f, 1));
    CHECK(oracle_beam_norm_residual_norm(rows, S, res, nw, nw, out, out2, T, H, 1e-6f, 1e-6f,
                                         0.5f, 2.0f, 1, 1));
    CHECK(oracle_beam_norm_residual_norm(rows, S, res, NULL, NULL, out, NULL, T, H, 0.0f,
                                         0.0f, 1.0f, 1.0f, 0, 0));
    CHECK(oracle_beam_moe_finalize_norm_residual_norm(e, T, K, H, w, res, nw, nw, out, out2, T,
                                                      1.5f, 1e-6f, 1e-6f, 1.0f, 1.0f, 1, 1));
    CHECK(oracle_beam_moe_finalize_norm_residual_norm(e, T, K, H, w, res, NULL, NULL, out,
                                                      NULL, 0, 1.0f, 0.0f, 0.0f, 1.0f, 1.0f,
                                                      0, 0));
    volatile uint16_t r = 0;
    for (int i = 0; i < 4096; ++i)
        r ^= oracle_round_to_bf16((double)(i - 2048) * 1.337e-40 * (i % 7 ? 1.0 : 1e80));
    free(rows); free(w); free(wb); free(idx); free(nw); free(out); free(out2); free(acc);
    free(e); free(res);
    printf("ok %u\n", (unsigned)r);
    return 0;
}
