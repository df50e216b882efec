/* A plain C99 caller of the all-reduce C ABI on the GPU: device memory from
 * the HIP runtime API, no Python and no torch.  R = 8 ranks of integer-valued
 * bf16 (exact sums), out of place and in place, each protocol and both LL flag
 * schemes; every output element is compared with the exact integer sum. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

int main(void)
{
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
