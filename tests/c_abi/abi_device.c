/* A plain C99 caller of the all-reduce C ABI on the GPU: device memory from
 * the HIP runtime API, no Python and no torch.  R = 8 ranks of integer-valued
 * bf16 (exact sums), out of place and in place, each protocol and both LL flag
 * schemes; every output element is compared with the exact integer sum.
 *
 * With --time it then prints the host's cost of eager calls from C: the mean
 * wall-clock time per call of 2000 back-to-back arAllReduce calls (after 200
 * untimed ones), up to a final device synchronisation, for the smallest call
 * (HB, one rank, 16 bytes) and for LL and HB at 8 ranks x 2 KiB. */
#define _POSIX_C_SOURCE 199309L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include <hip/hip_runtime_api.h>

#include "ar_allreduce.h"

enum { R = 8, N = 100003 };

/* bf16 bits of a small integer: the upper half of its binary32 bits (exact). */
static uint16_t bf16_of_int(int v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int check_hip(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        printf("FAIL: %s: %s\n", what, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

static double now_us(void)
{
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return t.tv_sec * 1e6 + t.tv_nsec * 1e-3;
}

/* Mean microseconds per eager call, or a negative value on an error. */
static double eager_us(void *const *sendp, void *const *recvp, size_t count, int nranks,
                       arProtocol_t proto, arComm_t comm)
{
    for (int i = 0; i < 200; ++i)
        if (arAllReduce((const void *const *)sendp, recvp, count, arBfloat16, arSum, nranks, proto,
                        comm, NULL) != arSuccess)
            return -1.0;
    if (hipDeviceSynchronize() != hipSuccess)
        return -1.0;
    const int calls = 2000;
    const double t0 = now_us();
    for (int i = 0; i < calls; ++i)
        if (arAllReduce((const void *const *)sendp, recvp, count, arBfloat16, arSum, nranks, proto,
                        comm, NULL) != arSuccess)
            return -1.0;
    if (hipDeviceSynchronize() != hipSuccess)
        return -1.0;
    return (now_us() - t0) / calls;
}

int main(int argc, char **argv)
{
    const int timing = argc > 1 && strcmp(argv[1], "--time") == 0;
    static uint16_t host[R][N], out[N], want[N];
    unsigned s = 12345u;
    for (int i = 0; i < N; ++i) {
        int sum = 0;
        for (int r = 0; r < R; ++r) {
            s = s * 1103515245u + 12345u;            /* a plain LCG: inputs only */
            const int v = (int)((s >> 16) % 9u) - 4; /* -4..4 */
            host[r][i] = bf16_of_int(v);
            sum += v;
        }
        want[i] = bf16_of_int(sum);
    }

    arComm_t comm = NULL;
    if (arCommCreate(&comm, 0, R, 1u << 20) != arSuccess) {
        printf("FAIL: arCommCreate\n");
        return 1;
    }
    void *sendp[R], *recvp[R];
    for (int r = 0; r < R; ++r)
        if (check_hip(hipMalloc(&sendp[r], N * 2), "hipMalloc") ||
            check_hip(hipMalloc(&recvp[r], N * 2), "hipMalloc"))
            return 1;

    const arProtocol_t protos[3] = {arProtoLL, arProtoHB, arProtoAuto};
    int failures = 0;
    /* both LL flag schemes: consumer clears (0, the default), sequence numbers (1) */
    for (int run = 0; run < 4; ++run) {
        const int inplace = run % 2, scheme = run / 2;
        if (arCommSetOption(comm, arOptLLFlagScheme, scheme) != arSuccess) {
            printf("FAIL: arCommSetOption(arOptLLFlagScheme, %d)\n", scheme);
            ++failures;
        }
        for (int p = 0; p < 3; ++p) {
            for (int r = 0; r < R; ++r)
                if (check_hip(hipMemcpy(sendp[r], host[r], N * 2, hipMemcpyHostToDevice), "H2D"))
                    return 1;
            void *const *dst = inplace ? sendp : recvp;
            const arResult_t rc = arAllReduce((const void *const *)sendp, dst, N, arBfloat16,
                                              arSum, R, protos[p], comm, NULL);
            arResult_t async = arSuccess;
            if (rc != arSuccess || check_hip(hipDeviceSynchronize(), "sync") ||
                arCommGetAsyncError(comm, &async) != arSuccess || async != arSuccess) {
                printf("FAIL: call %d/%d/%d: %s\n", p, inplace, scheme, arGetErrorString(rc));
                ++failures;
                continue;
            }
            for (int r = 0; r < R; ++r) {
                if (check_hip(hipMemcpy(out, dst[r], N * 2, hipMemcpyDeviceToHost), "D2H"))
                    return 1;
                if (memcmp(out, want, sizeof want) != 0) {
                    printf("FAIL: protocol %d in place %d scheme %d rank %d differs\n", p, inplace,
                           scheme, r);
                    ++failures;
                }
            }
        }
    }
    if (timing && failures == 0) {
        if (arCommSetOption(comm, arOptLLFlagScheme, 0) != arSuccess)
            ++failures;
        const double floor_us = eager_us(sendp, recvp, 8, 1, arProtoHB, comm);
        const double ll_us = eager_us(sendp, recvp, 1024, R, arProtoLL, comm);
        const double hb_us = eager_us(sendp, recvp, 1024, R, arProtoHB, comm);
        if (floor_us < 0 || ll_us < 0 || hb_us < 0) {
            printf("FAIL: timed calls\n");
            ++failures;
        } else {
            printf("eager us per call from C: hb_1rank_16B %.2f ll_8x2KiB %.2f hb_8x2KiB %.2f\n",
                   floor_us, ll_us, hb_us);
        }
    }
    for (int r = 0; r < R; ++r) {
        (void)hipFree(sendp[r]);
        (void)hipFree(recvp[r]);
    }
    if (arCommDestroy(comm) != arSuccess)
        ++failures;
    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
