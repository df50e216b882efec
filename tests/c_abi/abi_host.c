/* A plain C99 caller of the all-reduce C ABI, host side only: it needs no GPU.
 * Checks that the header compiles as C, that the library links, and the
 * answers the library gives before it touches a device. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ar_allreduce.h"

static int failures = 0;

static void expect(int cond, const char *what)
{
    if (!cond) {
        printf("FAIL: %s\n", what);
        ++failures;
    }
}

int main(void)
{
    expect(arGetVersion() == AR_VERSION, "arGetVersion");
    expect(strncmp(arGetErrorString(arSuccess), "arSuccess", 9) == 0, "error string");
    expect(strncmp(arGetErrorString(arTimeout), "arTimeout", 9) == 0, "timeout string");

    /* 16-byte aligned addresses that are never dereferenced */
    const void *send[2] = {(const void *)(uintptr_t)0x7f0000000000ull,
                           (const void *)(uintptr_t)0x7f0000001000ull};
    void *recv[2] = {(void *)(uintptr_t)0x7f0000002000ull, (void *)(uintptr_t)0x7f0000003000ull};
    expect(arAllReduce(send, recv, 1024, arBfloat16, arSum, 2, arProtoHB, NULL, NULL) ==
               arInvalidArgument, "NULL communicator");
    expect(arAllReduce(send, recv, 1024, (arDataType_t)7, arSum, 2, arProtoHB, NULL, NULL) ==
               arUnsupported, "unknown dtype");
    expect(arAllReduce(send, recv, 1024, arFloat32, arSum, 33, arProtoLL, NULL, NULL) ==
               arUnsupported, "33 ranks");
    expect(arAllReduce(send, recv, 0, arFloat16, arSum, 2, arProtoAuto, NULL, NULL) == arSuccess,
           "count 0 is a no-op");

    arComm_t comm = NULL;
    expect(arCommCreate(&comm, 0, 0, 1024) == arInvalidArgument && comm == NULL, "maxRanks 0");
    arTunedShape_t shape;
    expect(arCommGetTunedShape(NULL, arBfloat16, 8, arProtoHB, 4096, 0, &shape) ==
               arInvalidArgument, "tuned shape of a NULL communicator");
    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
