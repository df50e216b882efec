/* Drives every entry point of oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py).  Inputs are
 * integers in [-4, 4], so every sum is exact and is checked as such; the run
 * fails on the first sanitizer report or wrong sum. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_widen_bf16(uint16_t h);
float oracle_widen_fp16(uint16_t h);
uint16_t oracle_rne_bf16(float f);
uint16_t oracle_rne_fp16(float f);
int oracle_allreduce(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, int nthreads);
int oracle_allreduce_grouped(const void *const *send, void *const *recv, size_t count,
                             int dtype, int nranks, int group, int nthreads);
void oracle_rne_bf16_array(const float *in, uint16_t *out, size_t n, int nthreads);
void oracle_rne_fp16_array(const float *in, uint16_t *out, size_t n, int nthreads);
void oracle_widen_fp16_array(const uint16_t *in, float *out, size_t n);
double oracle_allreduce_timed(const void *const *send, void *const *recv, size_t count,
                              int dtype, int nranks, int nthreads);

static unsigned lcg = 7u;
static int next_int(void) /* -4..4 */
{
    lcg = lcg * 1103515245u + 12345u;
    return (int)((lcg >> 16) % 9u) - 4;
}

static int check(int dtype, int nranks, size_t count, int group, int nthreads)
{
    const size_t es = dtype == 2 ? 4 : 2;
    void *send[32], *recv[32];
    int *want = calloc(count ? count : 1, sizeof(int));
    for (int r = 0; r < nranks; ++r) {
        send[r] = malloc(count * es ? count * es : 1); /* exact sizes: overruns are caught */
        recv[r] = malloc(count * es ? count * es : 1);
        for (size_t i = 0; i < count; ++i) {
            const int v = next_int();
            want[i] += v;
            if (dtype == 0)
                ((uint16_t *)send[r])[i] = oracle_rne_bf16((float)v);
            else if (dtype == 1)
                ((uint16_t *)send[r])[i] = oracle_rne_fp16((float)v);
            else
                ((float *)send[r])[i] = (float)v;
        }
    }
    int rc = group > 0 ? oracle_allreduce_grouped((const void *const *)send, recv, count, dtype,
                                                  nranks, group, nthreads)
                       : oracle_allreduce((const void *const *)send, recv, count, dtype, nranks,
                                          nthreads);
    int bad = rc != 0;
    for (int r = 0; r < nranks && !bad; ++r)
        for (size_t i = 0; i < count && !bad; ++i) {
            float got = dtype == 0   ? oracle_widen_bf16(((uint16_t *)recv[r])[i])
                        : dtype == 1 ? oracle_widen_fp16(((uint16_t *)recv[r])[i])
                                     : ((float *)recv[r])[i];
            bad = got != (float)want[i];
        }
    if (!bad && group == 0) {
        const double t = oracle_allreduce_timed((const void *const *)send, recv, count, dtype,
                                                nranks, nthreads);
        bad = t < 0.0;
    }
    for (int r = 0; r < nranks; ++r) {
        free(send[r]);
        free(recv[r]);
    }
    free(want);
    if (bad)
        printf("FAIL: dtype %d nranks %d count %zu group %d\n", dtype, nranks, count, group);
    return bad;
}

int main(void)
{
    int failures = 0;
    const size_t counts[] = {1, 2, 3, 7, 9, 1023, 1025, 65541};
    const int ranks[] = {1, 2, 3, 5, 8, 13, 16, 32};
    for (int d = 0; d < 3; ++d)
        for (int a = 0; a < 8; ++a)
            for (int c = 0; c < 8; ++c)
                failures += check(d, ranks[a], counts[c], 0, 1 + (c % 4));
    const int groups[][2] = {{16, 8}, {32, 8}, {32, 4}, {8, 2}, {12, 4}, {6, 3}};
    for (int d = 0; d < 3; ++d)
        for (int g = 0; g < 6; ++g)
            for (int c = 0; c < 8; ++c)
                failures += check(d, groups[g][0], counts[c], groups[g][1], 2);
    /* bad arguments are refused, not read */
    failures += oracle_allreduce(NULL, NULL, 4, 7, 2, 1) == 0;
    failures += oracle_allreduce_grouped(NULL, NULL, 4, 0, 6, 4, 1) == 0;
    /* converters over a stretch of binary32 patterns, including NaN/inf/denormals */
    enum { M = 1 << 16 };
    float *f = malloc(M * sizeof(float));
    uint16_t *h = malloc(M * sizeof(uint16_t));
    float *w = malloc(M * sizeof(float));
    for (uint32_t i = 0; i < M; ++i) {
        const uint32_t u = i * 65537u + 12345u;
        memcpy(&f[i], &u, 4);
    }
    oracle_rne_bf16_array(f, h, M, 4);
    oracle_rne_fp16_array(f, h, M, 4);
    oracle_widen_fp16_array(h, w, M);
    free(f);
    free(h);
    free(w);
    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
