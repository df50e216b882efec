// api.hip -- the C ABI declared in include/ar_allreduce.h.
//
// Host side of each call: check the arguments without touching the device,
// pick the protocol's kernel, pack the rank table into the kernel arguments
// and enqueue one launch on the caller's stream.  Nothing here allocates,
// synchronises or records a memset, so calls can be captured into a HIP graph
// (the property the SGLang MSCCL++ all-reduce guide, blog.gitcode.com,
// section 1, gives as the reason MSCCL++ is used under CUDA Graph decode).
//
// The checks mirror the guards of that guide's section 4.3: SUM only, float /
// float16 / bfloat16 only, contiguous buffers (here: raw pointers, which must
// be 16-byte aligned for the 128-bit accesses).  The world-size guard (8, 16
// or 32 GPUs) becomes 1..32 simulated ranks.  A request the library does not
// serve returns arUnsupported so that the caller can fall back, as SGLang falls
// back to NCCL (sections 4.3 and 5).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "ar_internal.hpp"

namespace {

bool debug_enabled()
{
    static const bool on = [] {
        const char *v = getenv("AR_DEBUG");
        return v != nullptr && v[0] == '1';
    }();
    return on;
}

arResult_t reject(arResult_t r, const char *why)
{
    if (debug_enabled())
        fprintf(stderr, "[ar] %s: %s\n", arGetErrorString(r), why);
    return r;
}

size_t elem_bytes(arDataType_t dtype)
{
    return dtype == arFloat32 ? 4 : 2;
}

bool overlaps(uintptr_t a, uintptr_t b, size_t len)
{
    return a < b + len && b < a + len;
}

constexpr int64_t kDefaults[kOptionCount] = {
    2000000,  // arOptPollTimeoutUs
    0,        // arOptLLBlocksPerRank (auto)
    0,        // arOptHBBlocks (auto)
    1,        // arOptHBNonTemporal
    0,        // arOptDebugFlagSkew
    0,        // arOptHBUnroll (auto)
    0,        // arOptLLThreads (auto)
    0,        // arOptHBThreads (auto)
    1,        // arOptHBChunkLayout (interleaved tiles)
};

// Argument checks shared by every protocol.  No HIP call.
arResult_t validate(const void *const *sendbufs, void *const *recvbufs, size_t count,
                    arDataType_t dtype, arRedOp_t op, int nranks, arProtocol_t protocol)
{
    if (dtype != arBfloat16 && dtype != arFloat16 && dtype != arFloat32)
        return reject(arUnsupported, "dtype must be bf16, fp16 or fp32");
    if (op != arSum)
        return reject(arUnsupported, "only arSum is implemented");
    if (nranks < 1 || nranks > AR_MAX_RANKS)
        return reject(arUnsupported, "nranks must be in 1..32");
    if (protocol != arProtoLL && protocol != arProtoHB)
        return reject(arInvalidArgument, "unknown protocol");
    if (count == 0)
        return arSuccess;
    if (count > (SIZE_MAX / 8))
        return reject(arInvalidArgument, "count too large");
    if (sendbufs == nullptr || recvbufs == nullptr)
        return reject(arInvalidArgument, "NULL buffer array");
    const size_t len = count * elem_bytes(dtype);
    for (int r = 0; r < nranks; ++r) {
        const uintptr_t s = (uintptr_t)sendbufs[r], d = (uintptr_t)recvbufs[r];
        if (s == 0 || d == 0)
            return reject(arInvalidArgument, "NULL rank buffer");
        if ((s | d) & 15u)
            return reject(arInvalidArgument, "rank buffers must be 16-byte aligned");
        if (s > UINTPTR_MAX - len || d > UINTPTR_MAX - len)
            return reject(arInvalidArgument, "rank buffer wraps the address space");
    }
    // Receive buffers are written: they may not overlap each other, nor any
    // send buffer except their own rank's, and that one only exactly.
    for (int r = 0; r < nranks; ++r) {
        const uintptr_t d = (uintptr_t)recvbufs[r];
        for (int q = 0; q < nranks; ++q) {
            const uintptr_t s = (uintptr_t)sendbufs[q];
            if (q == r && s == d)
                continue;
            if (overlaps(d, s, len))
                return reject(arInvalidArgument,
                              "a receive buffer overlaps a send buffer other than its own");
            if (q != r && overlaps(d, (uintptr_t)recvbufs[q], len))
                return reject(arInvalidArgument, "receive buffers overlap");
        }
    }
    return arSuccess;
}

// RAII restore of the caller's current device.
struct DeviceGuard {
    int saved = -1;
    bool ok = false;
    explicit DeviceGuard(int device)
    {
        if (hipGetDevice(&saved) != hipSuccess)
            return;
        ok = hipSetDevice(device) == hipSuccess;
    }
    ~DeviceGuard()
    {
        if (saved >= 0)
            (void)hipSetDevice(saved);
    }
};

}  // namespace

extern "C" {

const char *arGetErrorString(arResult_t result)
{
    switch (result) {
    case arSuccess: return "arSuccess: no error";
    case arInvalidArgument: return "arInvalidArgument: invalid argument";
    case arUnsupported: return "arUnsupported: request not supported, use another all-reduce";
    case arInvalidUsage: return "arInvalidUsage: request exceeds the communicator's limits";
    case arHipError: return "arHipError: a HIP runtime call failed";
    case arTimeout: return "arTimeout: an LL packet wait timed out";
    case arInternalError: return "arInternalError: internal error";
    }
    return "unknown arResult_t";
}

int arGetVersion(void) { return AR_VERSION; }

arResult_t arCommCreate(arComm_t *comm, int device, int maxRanks, size_t maxLLBytesPerRank)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    *comm = nullptr;
    if (maxRanks < 1 || maxRanks > AR_MAX_RANKS)
        return reject(arInvalidArgument, "maxRanks must be in 1..32");
    if (maxLLBytesPerRank > ((size_t)1 << 34))
        return reject(arInvalidArgument, "maxLLBytesPerRank above 16 GiB");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        return reject(arHipError, "no such HIP device");

    DeviceGuard guard(device);
    if (!guard.ok)
        return reject(arHipError, "hipSetDevice failed");

    arComm *c = new (std::nothrow) arComm();
    if (c == nullptr)
        return arInternalError;
    c->device = device;
    c->max_ranks = maxRanks;
    c->max_ll_bytes = maxLLBytesPerRank;
    memcpy(c->opt, kDefaults, sizeof(kDefaults));

    int cus = 0, clock_khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, device) != hipSuccess ||
        cus <= 0 || clock_khz <= 0) {
        delete c;
        return reject(arHipError, "device attribute query failed");
    }
    c->cu_count = cus;
    c->wall_clock_khz = (uint64_t)clock_khz;

    // Packets: 8 bytes for each 4 payload bytes; round each rank's region up
    // to a whole number of 256-byte lines.
    const uint64_t words = (maxLLBytesPerRank + 3) / 4;
    c->pkt_stride = (words + 31) / 32 * 32;
    const size_t pkt_bytes = (size_t)maxRanks * c->pkt_stride * sizeof(uint64_t);
    if (hipMalloc((void **)&c->ctrl, 256) != hipSuccess) {
        delete c;
        return reject(arHipError, "hipMalloc of control words failed");
    }
    c->pkts = nullptr;
    if (pkt_bytes > 0 && hipMalloc((void **)&c->pkts, pkt_bytes) != hipSuccess) {
        (void)hipFree(c->ctrl);
        delete c;
        return reject(arHipError, "hipMalloc of LL packet memory failed");
    }
    if (hipMemset(c->ctrl, 0, 256) != hipSuccess ||
        (pkt_bytes > 0 && hipMemset(c->pkts, 0, pkt_bytes) != hipSuccess) ||
        ar::query_ll_residency(c) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(c->pkts);
        (void)hipFree(c->ctrl);
        delete c;
        return reject(arHipError, "communicator set-up failed");
    }
    *comm = c;
    return arSuccess;
}

arResult_t arCommDestroy(arComm_t comm)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    DeviceGuard guard(comm->device);
    arResult_t r = arSuccess;
    if (comm->pkts != nullptr && hipFree(comm->pkts) != hipSuccess)
        r = arHipError;
    if (comm->ctrl != nullptr && hipFree(comm->ctrl) != hipSuccess)
        r = arHipError;
    delete comm;
    return r;
}

arResult_t arCommReset(arComm_t comm, arStream_t stream)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != comm->device)
        return reject(arInvalidUsage, "the communicator's device is not the current device");
    if (ar::launch_reset(comm, (hipStream_t)stream) != hipSuccess)
        return reject(arHipError, "reset launch failed");
    return arSuccess;
}

arResult_t arCommGetAsyncError(arComm_t comm, arResult_t *asyncError)
{
    if (comm == nullptr || asyncError == nullptr)
        return reject(arInvalidArgument, "NULL argument");
    DeviceGuard guard(comm->device);
    uint32_t word = 0;
    if (!guard.ok || hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&word, comm->ctrl + 0, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return reject(arHipError, "reading the error word failed");
    *asyncError = word == 0 ? arSuccess : (arResult_t)word;
    return arSuccess;
}

arResult_t arCommSetOption(arComm_t comm, arOption_t option, int64_t value)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    bool ok = false;
    switch (option) {
    case arOptPollTimeoutUs: ok = value >= 1 && value <= 600000000; break;
    case arOptLLBlocksPerRank: ok = value >= 0 && value <= 65536; break;
    case arOptHBBlocks: ok = value >= 0 && value <= (1 << 20); break;
    case arOptHBNonTemporal: ok = value == 0 || value == 1; break;
    case arOptDebugFlagSkew: ok = value >= 0 && value <= 65535; break;
    case arOptHBUnroll: ok = value == 0 || value == 1 || value == 2 || value == 4; break;
    case arOptLLThreads:
        ok = value == 0 || value == 64 || value == 128 || value == 256 || value == 512 ||
             value == 1024;
        break;
    case arOptHBThreads: ok = value >= 0 && value <= 1024 && value % 64 == 0; break;
    case arOptHBChunkLayout: ok = value == 0 || value == 1; break;
    default: return reject(arInvalidArgument, "unknown option");
    }
    if (!ok)
        return reject(arInvalidArgument, "option value out of range");
    comm->opt[option] = value;
    return arSuccess;
}

arResult_t arCommGetOption(arComm_t comm, arOption_t option, int64_t *value)
{
    if (comm == nullptr || value == nullptr)
        return reject(arInvalidArgument, "NULL argument");
    if ((int)option < 0 || (int)option >= kOptionCount)
        return reject(arInvalidArgument, "unknown option");
    *value = comm->opt[option];
    return arSuccess;
}

arResult_t arAllReduce(const void *const *sendbufs, void *const *recvbufs, size_t count,
                       arDataType_t dtype, arRedOp_t op, int nranks, arProtocol_t protocol,
                       arComm_t comm, arStream_t stream)
{
    arResult_t r = validate(sendbufs, recvbufs, count, dtype, op, nranks, protocol);
    if (r != arSuccess || count == 0)
        return r;
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    if (protocol == arProtoLL) {
        if (nranks > comm->max_ranks)
            return reject(arInvalidUsage, "nranks above the communicator's maxRanks");
        if (count * elem_bytes(dtype) > comm->max_ll_bytes)
            return reject(arInvalidUsage, "message above the communicator's maxLLBytesPerRank");
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != comm->device)
        return reject(arInvalidUsage, "the communicator's device is not the current device");

    const hipError_t e =
        protocol == arProtoLL
            ? ar::launch_ll(sendbufs, recvbufs, count, (int)dtype, nranks, comm, (hipStream_t)stream)
            : ar::launch_hb(sendbufs, recvbufs, count, (int)dtype, nranks, comm, (hipStream_t)stream);
    if (e != hipSuccess)
        return reject(arHipError, hipGetErrorString(e));
    return arSuccess;
}

}  // extern "C"
