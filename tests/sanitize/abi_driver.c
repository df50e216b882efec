/* Drives the host side of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer with no GPU (built by tests/test_sanitizers.py):
 * error strings, every entry point with a NULL communicator, arCommCreate with
 * no usable device, and a few thousand randomised arAllReduce argument sets
 * whose pointer arrays are heap blocks of exactly nranks entries, so a read
 * past them is reported.  Pointers themselves are never dereferenced. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ar_allreduce.h"

static unsigned lcg = 99u;
static unsigned next_u(void)
{
    lcg = lcg * 1103515245u + 12345u;
    return lcg >> 8;
}

int main(void)
{
    int failures = 0;
    for (int r = -1; r <= 8; ++r)
        failures += arGetErrorString((arResult_t)r) == NULL;
    failures += arGetVersion() != AR_VERSION;

    arComm_t comm = NULL;
    const arResult_t cr = arCommCreate(&comm, 0, 8, 1u << 20);
    failures += cr == arSuccess; /* no GPU here */
    failures += arCommDestroy(NULL) != arInvalidArgument;
    failures += arCommReset(NULL, NULL) != arInvalidArgument;
    failures += arCommSetOption(NULL, arOptHBBlocks, 1) != arInvalidArgument;
    int64_t v = 0;
    failures += arCommGetOption(NULL, arOptHBBlocks, &v) != arInvalidArgument;
    arResult_t ae = arSuccess;
    failures += arCommGetAsyncError(NULL, &ae) != arInvalidArgument;
    failures += arCommTune(NULL, arBfloat16, 8, 1u << 20, NULL) != arInvalidArgument;
    arTunedShape_t shape;
    failures += arCommGetTunedShape(NULL, arBfloat16, 8, arProtoHB, 4096, 0, &shape) !=
                arInvalidArgument;

    for (int it = 0; it < 5000; ++it) {
        const int nranks = (int)(next_u() % 35u);            /* 0..34 */
        const size_t count = (next_u() % 4u == 0) ? 0 : (size_t)(next_u() % 70000u);
        const int dtype = (int)(next_u() % 9u) - 1;           /* -1 and 3..7 are invalid */
        const int proto = (int)(next_u() % 9u) - 1;           /* -1 and 3..7 are invalid */
        const int op = next_u() % 10u == 0 ? (int)(next_u() % 5u) - 1 : 0;
        const int n = nranks > 0 ? nranks : 1;
        const void **send = malloc(sizeof(void *) * (size_t)n);
        void **recv = malloc(sizeof(void *) * (size_t)n);
        for (int r = 0; r < n; ++r) {
            const uintptr_t base = 0x7f0000000000ull + (uintptr_t)(next_u() % 12u) * (1u << 20);
            const uintptr_t off = (next_u() % 8u == 0) ? 8 : 0;
            send[r] = (const void *)(base + off);
            recv[r] = next_u() % 3u == 0 ? (void *)(base + off)
                                         : (void *)(0x7f8000000000ull +
                                                    (uintptr_t)(next_u() % 12u) * (1u << 20));
            if (next_u() % 50u == 0)
                send[r] = NULL;
        }
        const arResult_t res = arAllReduce(send, recv, count, (arDataType_t)dtype,
                                           (arRedOp_t)op, nranks, (arProtocol_t)proto, NULL,
                                           NULL);
        /* with no communicator nothing can succeed except an empty valid call */
        if (res == arSuccess && count != 0)
            ++failures;
        free(send);
        free(recv);
    }
    if (failures == 0)
        printf("ok\n");
    else
        printf("FAIL: %d\n", failures);
    return failures == 0 ? 0 : 1;
}
