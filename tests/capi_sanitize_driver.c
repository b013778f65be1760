/*
 * Drives the C ABI's host code (argument validation and the launch plan)
 * under AddressSanitizer and UndefinedBehaviorSanitizer, with the recording
 * stand-in of tests/capi_host_stub.cpp in place of the GPU launcher.
 * tests/test_capi_sanitized.py builds it with capi.cpp and the stand-in and
 * feeds it the same cases as the host validation tests.
 *
 * Input, one call per line on stdin:
 *   <entry point> <argument> ...   every argument of the C prototype in order;
 *                                  pointers as integers (0 is NULL; they are
 *                                  never dereferenced), floats in C syntax
 *   reset                          forget the recorded launches
 *   fail <code>                    the next launch returns <code>
 * Output, one line per call:
 *   <status> <12 values of the stand-in's record> <1 if mf_last_error_message
 *   is non-empty, else 0>
 * Exit status 0 once every line has been run, 2 on a malformed line.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_finalize.h"

void mf_test_reset(void);
void mf_test_fail_next_launch(int code);
void mf_test_record(int64_t *out);

/* Argument kinds of each entry point: p pointer, L int64_t, i int32_t, f float. */
static const struct {
    const char *name;
    const char *kinds;
} kSigs[] = {
    {"moe_finalize_rmsnorm", "pLLpippLLiiffip"},
    {"moe_finalize", "pLLpippLiip"},
    {"beam_moe_finalize", "pLiipLpLpffip"},
    {"mf_rmsnorm", "pLppLiffip"},
    {"beam_moe_finalize_norm_residual_norm", "pLiipLpppppLfffffiip"},
    {"beam_norm_residual_norm", "pLpppppLiffffiip"},
};

#define MAX_ARGS 24

typedef union {
    void *p;
    int64_t L;
    int32_t i;
    float f;
} arg_t;

static int parse_args(const char *kinds, char *rest, arg_t *a)
{
    int n = (int)strlen(kinds);
    for (int k = 0; k < n; ++k) {
        char *tok = strtok(k == 0 ? rest : NULL, " \t\r\n");
        if (!tok)
            return -1;
        char *end = NULL;
        switch (kinds[k]) {
        case 'p':
            a[k].p = (void *)(uintptr_t)strtoull(tok, &end, 0);
            break;
        case 'L':
            a[k].L = (int64_t)strtoll(tok, &end, 0);
            break;
        case 'i':
            a[k].i = (int32_t)strtol(tok, &end, 0);
            break;
        case 'f':
            a[k].f = strtof(tok, &end);
            break;
        default:
            return -1;
        }
        if (!end || *end)
            return -1;
    }
    return strtok(NULL, " \t\r\n") ? -1 : 0;
}

static int call(int which, const arg_t *a)
{
    switch (which) {
    case 0:
        return moe_finalize_rmsnorm(a[0].p, a[1].L, a[2].L, a[3].p, a[4].i, (const int32_t *)a[5].p,
                                    a[6].p, a[7].p, a[8].L, a[9].i, a[10].i, a[11].f, a[12].f,
                                    a[13].i, a[14].p);
    case 1:
        return moe_finalize(a[0].p, a[1].L, a[2].L, a[3].p, a[4].i, (const int32_t *)a[5].p,
                            a[6].p, a[7].L, a[8].i, a[9].i, a[10].p);
    case 2:
        return beam_moe_finalize(a[0].p, a[1].L, a[2].i, a[3].i, (const float *)a[4].p, a[5].L,
                                 a[6].p, a[7].L, a[8].p, a[9].f, a[10].f, a[11].i, a[12].p);
    case 3:
        return mf_rmsnorm(a[0].p, a[1].L, a[2].p, a[3].p, a[4].L, a[5].i, a[6].f, a[7].f,
                          a[8].i, a[9].p);
    case 4:
        return beam_moe_finalize_norm_residual_norm(
            a[0].p, a[1].L, a[2].i, a[3].i, (const float *)a[4].p, a[5].L, a[6].p, a[7].p, a[8].p,
            a[9].p, a[10].p, a[11].L, a[12].f, a[13].f, a[14].f, a[15].f, a[16].f, a[17].i,
            a[18].i, a[19].p);
    case 5:
        return beam_norm_residual_norm(a[0].p, a[1].L, a[2].p, a[3].p, a[4].p, a[5].p, a[6].p,
                                       a[7].L, a[8].i, a[9].f, a[10].f, a[11].f, a[12].f,
                                       a[13].i, a[14].i, a[15].p);
    }
    return -1;
}

int main(void)
{
    char line[4096];
    int lineno = 0;
    mf_test_reset();
    while (fgets(line, sizeof line, stdin)) {
        ++lineno;
        char *name = strtok(line, " \t\r\n");
        if (!name)
            continue;
        if (strcmp(name, "reset") == 0) {
            mf_test_reset();
            continue;
        }
        if (strcmp(name, "fail") == 0) {
            char *tok = strtok(NULL, " \t\r\n");
            if (!tok)
                goto bad;
            mf_test_fail_next_launch((int)strtol(tok, NULL, 0));
            continue;
        }
        int which = -1;
        for (int k = 0; k < (int)(sizeof kSigs / sizeof kSigs[0]); ++k)
            if (strcmp(name, kSigs[k].name) == 0)
                which = k;
        if (which < 0)
            goto bad;
        arg_t a[MAX_ARGS];
        memset(a, 0, sizeof a);
        if (parse_args(kSigs[which].kinds, name + strlen(name) + 1, a) != 0)
            goto bad;
        int status = call(which, a);
        int64_t rec[14];
        mf_test_record(rec);
        printf("%d", status);
        for (int k = 0; k < 14; ++k)
            printf(" %lld", (long long)rec[k]);
        const char *msg = mf_last_error_message();
        printf(" %d\n", msg && msg[0] ? 1 : 0);
        if (strcmp(mf_status_string(status), "") == 0)
            goto bad;
    }
    return 0;
bad:
    fprintf(stderr, "malformed line %d\n", lineno);
    return 2;
}
