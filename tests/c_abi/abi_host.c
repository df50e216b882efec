/* A plain C99 caller of the all-reduce C ABI, host side only: it needs no GPU.
 * Checks that the header compiles as C, that the library links, and the
 * answers the library gives before it touches a device. */
#include <stddef.h>
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

int main(int argc, char **argv)
{
    /* With "layout": print the C layout of the ABI's struct, for the binding's
     * mirror of it to be checked against. */
    if (argc > 1 && strcmp(argv[1], "layout") == 0) {
        printf("arTunedShape_t %zu tuned %zu threads %zu blocks %zu packetBytes %zu "
               "nonTemporal %zu us %zu\n",
               sizeof(arTunedShape_t), offsetof(arTunedShape_t, tuned),
               offsetof(arTunedShape_t, threads), offsetof(arTunedShape_t, blocks),
               offsetof(arTunedShape_t, packetBytes), offsetof(arTunedShape_t, nonTemporal),
               offsetof(arTunedShape_t, us));
        printf("arLaunchInfo_t %zu protocol %zu kernels %zu grid %zu threads %zu "
               "packetBytes %zu nonTemporal %zu nodeRanks %zu staged %zu packetPayloadBytes %zu\n",
               sizeof(arLaunchInfo_t), offsetof(arLaunchInfo_t, protocol),
               offsetof(arLaunchInfo_t, kernels), offsetof(arLaunchInfo_t, grid),
               offsetof(arLaunchInfo_t, threads), offsetof(arLaunchInfo_t, packetBytes),
               offsetof(arLaunchInfo_t, nonTemporal), offsetof(arLaunchInfo_t, nodeRanks),
               offsetof(arLaunchInfo_t, staged), offsetof(arLaunchInfo_t, packetPayloadBytes));
        printf("arResult_t %zu arDataType_t %zu arRedOp_t %zu arProtocol_t %zu arOption_t %zu\n",
               sizeof(arResult_t), sizeof(arDataType_t), sizeof(arRedOp_t),
               sizeof(arProtocol_t), sizeof(arOption_t));
        return 0;
    }
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
    arLaunchInfo_t info;
    expect(arCommGetLastLaunch(NULL, &info) == arInvalidArgument,
           "last launch of a NULL communicator");
    if (failures == 0)
        printf("ok\n");
    return failures == 0 ? 0 : 1;
}
