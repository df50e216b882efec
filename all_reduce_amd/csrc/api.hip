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

#include <mutex>
#include <new>
#include <vector>

#include "ar_internal.hpp"

// Device scratch of arAllReduceNoAlloc: the node partials of its staged
// two-level form, one copy per GPU, held until the process ends.  In host
// code `scratch` is only a stand-in for the symbol: its device address is
// looked up once per device with hipGetSymbolAddress (noalloc_device below)
// and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[AR_NOALLOC_SCRATCH_BYTES];

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

// The integer a caller passed for an enum argument.  A C caller may pass any
// int, and reading a value outside the enumerators' range as the C++ enum type
// is undefined, so entry points read enum arguments as int, validate them, and
// convert back only values known to be valid.
template <typename E>
int raw(const E &e)
{
    static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

size_t elem_bytes(arDataType_t dtype)
{
    return dtype == arFloat32 ? 4 : 2;
}

bool overlaps(uintptr_t a, uintptr_t b, size_t len)
{
    return a < b + len && b < a + len;
}

// [a, a + la) and [b, b + lb) share a byte.
bool ranges_overlap(uintptr_t a, size_t la, uintptr_t b, size_t lb)
{
    return a < b + lb && b < a + la;
}

constexpr int64_t kDefaults[kOptionCount] = {
    2000000,  // arOptPollTimeoutUs
    0,        // arOptLLBlocksPerRank (auto)
    0,        // arOptHBBlocks (auto)
    -1,       // arOptHBNonTemporal (tuned, else non-temporal)
    0,        // arOptDebugFlagSkew
    0,        // arOptHBUnroll (auto)
    0,        // arOptLLThreads (auto)
    0,        // arOptHBThreads (auto)
    1,        // arOptHBChunkLayout (interleaved tiles)
    0,        // arOptNodeRanks (flat order)
    0,        // arOptLLPacketBytes (tuned, else by size)
    0,        // arOptHBStaged (fused)
    0,        // arOptLLFlagScheme (cleared)
    0,        // arOptDebugSeqStart
    0,        // arOptTuneFreshInputs (unchanged inputs)
    -1,       // arOptLLDense (by size)
};

// Argument checks shared by every protocol.  No HIP call.
arResult_t validate(const void *const *sendbufs, void *const *recvbufs, size_t count,
                    int dtype, int op, int nranks, int protocol)
{
    if (dtype != arBfloat16 && dtype != arFloat16 && dtype != arFloat32)
        return reject(arUnsupported, "dtype must be bf16, fp16 or fp32");
    if (op != arSum)
        return reject(arUnsupported, "only arSum is implemented");
    if (nranks < 1 || nranks > AR_MAX_RANKS)
        return reject(arUnsupported, "nranks must be in 1..32");
    if (protocol != arProtoLL && protocol != arProtoHB && protocol != arProtoAuto)
        return reject(arInvalidArgument, "unknown protocol");
    if (count == 0)
        return arSuccess;
    if (count > (SIZE_MAX / 8))
        return reject(arInvalidArgument, "count too large");
    if (sendbufs == nullptr || recvbufs == nullptr)
        return reject(arInvalidArgument, "NULL buffer array");
    const size_t len = count * elem_bytes((arDataType_t)dtype);
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

// Size bucket of a message: ceil(log2(bytes per rank)).
int bucket_of(size_t bytes)
{
    int b = 0;
    while (b < ar::kBuckets - 1 && ((size_t)1 << b) < bytes)
        ++b;
    return b;
}

bool ll_possible(const arComm *comm, int nranks, size_t bytes)
{
    return nranks <= comm->max_ranks && bytes <= comm->max_ll_bytes;
}

// The protocol a call runs: arProtoAuto resolves to the tuned faster one,
// and to LL only where LL can run the call (`ll_allowed`).
arProtocol_t resolve_protocol(const arComm *comm, arDataType_t dtype, int nranks, size_t bytes,
                              int in_place, arProtocol_t protocol, bool ll_allowed)
{
    if (protocol != arProtoAuto)
        return protocol;
    const int b = bucket_of(bytes);
    const ar::TunedShape &ll = comm->tuned[dtype][nranks][arProtoLL][in_place][b];
    const ar::TunedShape &hb = comm->tuned[dtype][nranks][arProtoHB][in_place][b];
    if (ll_allowed && ll_possible(comm, nranks, bytes) && ll.valid && (!hb.valid || ll.us < hb.us))
        return arProtoLL;
    return arProtoHB;
}

// The HB launchers' view of a communicator: its compute units and HB
// options, and its launch record.
ar::HBConfig hb_config(const arComm *comm)
{
    return {comm->cu_count, (int)comm->opt[arOptHBUnroll], comm->opt[arOptHBChunkLayout] == 1,
            &comm->last};
}

// Whether an LL call takes the three-element packets (ll_dense.hip): 16-bit
// types in the flat order, the cleared scheme and 8-byte packets only; then
// arOptLLDense, or by default from the size where they measured faster.
bool ll_dense(const arComm *comm, arDataType_t dtype, int nranks, size_t bytes, int pkt_bytes,
              int scheme, int group)
{
    if (dtype == arFloat32 || group != 0 || scheme != ar::kSchemeCleared || pkt_bytes == 16)
        return false;
    const int64_t o = comm->opt[arOptLLDense];
    return o < 0 ? bytes >= ar::ll_dense_from_bytes(nranks) : o == 1;
}

hipError_t launch(const void *const *send, void *const *recv, size_t count, arDataType_t dtype,
                  int nranks, arProtocol_t proto, const arComm *comm, int threads,
                  uint64_t blocks, int pkt_bytes, int scheme, int group, bool nt,
                  hipStream_t stream)
{
    if (proto == arProtoLL && ll_dense(comm, dtype, nranks, count * elem_bytes(dtype), pkt_bytes,
                                       scheme, group))
        return ar::launch_ll_dense(send, recv, count, (int)dtype, nranks, comm, threads, blocks,
                                   stream);
    return proto == arProtoLL
               ? ar::launch_ll(send, recv, count, (int)dtype, nranks, comm, threads, blocks,
                               pkt_bytes, scheme, group, stream)
               : ar::launch_hb(send, recv, count, (int)dtype, nranks, hb_config(comm), threads,
                               blocks, group, nt, stream);
}

// The tuner's input rewrite (arOptTuneFreshInputs): the first `vecs` 16-byte
// vectors of each of `nranks` regions `stride` bytes apart get a fixed
// pattern, one rank per grid row, with ordinary vector stores (a kernel, not
// a memset node, since it is captured into graphs).
__global__ __launch_bounds__(256) void tune_fill(char *base, uint64_t stride, uint64_t vecs)
{
    uint4 *p = reinterpret_cast<uint4 *>(base + (uint64_t)blockIdx.y * stride);
    const uint4 v = make_uint4(0x3c3c3c3cu, 0x3c3c3c3cu, 0x3c3c3c3cu, 0x3c3c3c3cu);
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < vecs;
         i += (uint64_t)gridDim.x * 256u)
        p[i] = v;
}

struct TuneFill {
    char *base;       // nullptr: no rewrite
    uint64_t stride;  // bytes between ranks' regions
    uint64_t vecs;    // 16-byte vectors rewritten per rank
    int nranks;
};

hipError_t launch_fill(const TuneFill &f, hipStream_t cs)
{
    if (f.vecs == 0)
        return hipSuccess;
    uint64_t gx = (f.vecs + 255) / 256;
    if (gx > 1024)
        gx = 1024;
    hipLaunchKernelGGL(tune_fill, dim3((uint32_t)gx, (uint32_t)f.nranks), dim3(256), 0, cs, f.base,
                       f.stride, f.vecs);
    return hipGetLastError();
}

// Per-call time of one tuning candidate: `calls` launches captured into a HIP
// graph on the tuner's private stream, one warm-up replay, then the best of
// two timed replays.  Graph replay is how latency-sensitive callers run the
// library; timing eager launches would measure the host's launch rate instead
// (about 10 us per call, above the kernel time of every message up to a few
// hundred KiB per rank).  With `fill.base` set, each launch is preceded by the
// input rewrite; with `call` false, only the rewrites are timed.
hipError_t time_candidate(const void *const *send, void *const *dst, size_t count,
                          arDataType_t dtype, int nranks, arProtocol_t proto, const arComm *comm,
                          int threads, uint64_t blocks, int pkt_bytes, int scheme, bool nt,
                          const TuneFill &fill, bool call, int calls, hipStream_t cs,
                          hipEvent_t e0, hipEvent_t e1, float *us)
{
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess)
        return e;
    hipError_t le = hipSuccess;
    for (int i = 0; i < calls && le == hipSuccess; ++i) {
        if (fill.base != nullptr)
            le = launch_fill(fill, cs);
        if (le == hipSuccess && call)
            le = launch(send, dst, count, dtype, nranks, proto, comm, threads, blocks, pkt_bytes,
                        scheme, 0, nt, cs);
    }
    e = hipStreamEndCapture(cs, &graph);  // always ends the capture
    if (le != hipSuccess)
        e = le;
    if (e == hipSuccess)
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e == hipSuccess)
        e = hipGraphLaunch(exec, cs);
    float best = 0.0f;
    for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
        e = hipEventRecord(e0, cs);
        if (e == hipSuccess)
            e = hipGraphLaunch(exec, cs);
        if (e == hipSuccess)
            e = hipEventRecord(e1, cs);
        if (e == hipSuccess)
            e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, e0, e1);
        const float t = ms * 1000.0f / (float)calls;
        if (rep == 0 || t < best)
            best = t;
    }
    if (exec != nullptr)
        (void)hipGraphExecDestroy(exec);
    if (graph != nullptr)
        (void)hipGraphDestroy(graph);
    *us = best;
    return e;
}

// Ranks per simulated node when a hierarchical order is in force, else 0.
int hierarchy_group(const arComm *comm, int nranks)
{
    const int g = (int)comm->opt[arOptNodeRanks];
    return g > 1 && g < nranks ? g : 0;
}

// Per-device state of arAllReduceNoAlloc: the device address of `scratch` and
// the compute-unit count, found once per device with that device current.
// Neither lookup allocates.
constexpr int kNoAllocMaxDevices = 64;
struct NoAllocDevice {
    bool ready;
    void *scratch;
    int cu_count;
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kNoAllocMaxDevices];

arResult_t noalloc_device(int device, NoAllocDevice *out)
{
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoAllocDevice &d = g_noalloc[device];
    if (!d.ready) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return reject(arHipError, "hipGetSymbolAddress of the no-alloc scratch failed");
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) !=
                hipSuccess || cus <= 0)
            return reject(arHipError, "device attribute query failed");
        d.scratch = ptr;
        d.cu_count = cus;
        d.ready = true;
    }
    *out = d;
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
    switch (raw(result)) {
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
    c->last = {-1, 0, 0, 0, 0, 0, 0, 0, 0};
    c->ws = nullptr;
    c->ws_bytes = 0;

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
    // to a whole number of 512-byte groups (the sequenced scheme's unit), with
    // one 4-byte sequence entry per group and rank region.
    const uint64_t words = (maxLLBytesPerRank + 3) / 4;
    c->pkt_stride = (words + 63) / 64 * 64;
    const size_t pkt_bytes = (size_t)maxRanks * c->pkt_stride * sizeof(uint64_t);
    c->seq_words = c->pkt_stride / 64 * (uint64_t)maxRanks;
    const size_t seq_bytes = c->seq_words * sizeof(uint32_t);
    c->ll16_ok = pkt_bytes < ((size_t)1 << 32);
    if (hipMalloc((void **)&c->ctrl, 256) != hipSuccess) {
        delete c;
        return reject(arHipError, "hipMalloc of control words failed");
    }
    c->pkts = nullptr;
    c->seq = nullptr;
    if ((pkt_bytes > 0 && hipMalloc((void **)&c->pkts, pkt_bytes) != hipSuccess) ||
        (seq_bytes > 0 && hipMalloc((void **)&c->seq, seq_bytes) != hipSuccess)) {
        (void)hipFree(c->pkts);
        (void)hipFree(c->ctrl);
        delete c;
        return reject(arHipError, "hipMalloc of LL packet memory failed");
    }
    if (hipMemset(c->ctrl, 0, 256) != hipSuccess ||
        (pkt_bytes > 0 && hipMemset(c->pkts, 0, pkt_bytes) != hipSuccess) ||
        (seq_bytes > 0 && hipMemset(c->seq, 0, seq_bytes) != hipSuccess) ||
        ar::query_ll_residency(c) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(c->seq);
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
    if (comm->seq != nullptr && hipFree(comm->seq) != hipSuccess)
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

arResult_t arCommSetOption(arComm_t comm, arOption_t option_arg, int64_t value)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    const int option = raw(option_arg);
    bool ok = false;
    switch (option) {
    case arOptPollTimeoutUs: ok = value >= 1 && value <= 600000000; break;
    case arOptLLBlocksPerRank: ok = value >= 0 && value <= 65536; break;
    case arOptHBBlocks: ok = value >= 0 && value <= (1 << 20); break;
    case arOptHBNonTemporal: ok = value >= -1 && value <= 1; break;
    case arOptDebugFlagSkew: ok = value >= 0 && value <= 65535; break;
    case arOptHBUnroll: ok = value == 0 || value == 1 || value == 2 || value == 4; break;
    case arOptLLThreads:
        ok = value == 0 || value == 64 || value == 128 || value == 256 || value == 512 ||
             value == 1024;
        break;
    case arOptHBThreads: ok = value >= 0 && value <= 1024 && value % 64 == 0; break;
    case arOptHBChunkLayout: ok = value == 0 || value == 1; break;
    case arOptNodeRanks: ok = value >= 0 && value <= AR_MAX_RANKS; break;
    case arOptHBStaged: ok = value == 0 || value == 1; break;
    case arOptLLFlagScheme: ok = value == 0 || value == 1; break;
    case arOptDebugSeqStart: ok = value >= 0 && value <= 0xffffffffLL; break;
    case arOptTuneFreshInputs: ok = value == 0 || value == 1; break;
    case arOptLLDense: ok = value >= -1 && value <= 1; break;
    case arOptLLPacketBytes:
        if (value == 16 && !comm->ll16_ok)
            return reject(arUnsupported, "16-byte packets need packet memory below 4 GiB");
        ok = value == 0 || value == 8 || value == 16;
        break;
    default: return reject(arInvalidArgument, "unknown option");
    }
    if (!ok)
        return reject(arInvalidArgument, "option value out of range");
    comm->opt[option] = value;
    return arSuccess;
}

arResult_t arCommSetWorkspace(arComm_t comm, void *workspace, size_t bytes)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    if ((workspace == nullptr) != (bytes == 0))
        return reject(arInvalidArgument, "a workspace needs both a pointer and a size");
    if (((uintptr_t)workspace & 255u) != 0)
        return reject(arInvalidArgument, "the workspace must be 256-byte aligned");
    if (workspace != nullptr && (uintptr_t)workspace > UINTPTR_MAX - bytes)
        return reject(arInvalidArgument, "the workspace wraps the address space");
    comm->ws = workspace;
    comm->ws_bytes = bytes;
    return arSuccess;
}

arResult_t arCommGetOption(arComm_t comm, arOption_t option_arg, int64_t *value)
{
    if (comm == nullptr || value == nullptr)
        return reject(arInvalidArgument, "NULL argument");
    const int option = raw(option_arg);
    if (option < 0 || option >= kOptionCount)
        return reject(arInvalidArgument, "unknown option");
    *value = comm->opt[option];
    return arSuccess;
}

arResult_t arAllReduce(const void *const *sendbufs, void *const *recvbufs, size_t count,
                       arDataType_t dtype_arg, arRedOp_t op_arg, int nranks,
                       arProtocol_t protocol_arg, arComm_t comm, arStream_t stream)
{
    arResult_t r = validate(sendbufs, recvbufs, count, raw(dtype_arg), raw(op_arg), nranks,
                            raw(protocol_arg));
    if (r != arSuccess || count == 0)
        return r;
    const arDataType_t dtype = (arDataType_t)raw(dtype_arg);
    const arProtocol_t protocol = (arProtocol_t)raw(protocol_arg);
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    const size_t bytes = count * elem_bytes(dtype);
    const int group = hierarchy_group(comm, nranks);
    int in_place = 1;
    for (int r = 0; r < nranks; ++r)
        in_place &= sendbufs[r] == recvbufs[r] ? 1 : 0;
    if (group != 0 && nranks % group != 0)
        return reject(arInvalidUsage, "nranks is not a multiple of arOptNodeRanks");
    // The hierarchical order is built into the fused HB kernel, the LL kernel
    // of the cleared flag scheme and the staged two-level HB form; the
    // sequenced LL ablation keeps the flat order.
    const bool staged = comm->opt[arOptHBStaged] != 0;
    const bool seq_ll = comm->opt[arOptLLFlagScheme] == ar::kSchemeSequenced;
    const arProtocol_t proto = resolve_protocol(comm, dtype, nranks, bytes, in_place, protocol,
                                                group == 0 || !seq_ll);
    if (group != 0 && proto == arProtoLL && seq_ll)
        return reject(arUnsupported, "the sequenced LL scheme sums in the flat order only");
    const bool two_level = group != 0 && proto == arProtoHB && staged;
    if (two_level) {
        const uint64_t need = ar::hier_workspace_bytes(count, nranks / group);
        if (need == UINT64_MAX)
            return reject(arInvalidArgument, "message too large for the two-level form");
        if (comm->ws == nullptr || comm->ws_bytes < need)
            return reject(arInvalidUsage, "the staged two-level form needs a workspace of "
                                          "(nranks / arOptNodeRanks) * roundup(count * 4, 256) "
                                          "bytes (arCommSetWorkspace)");
        const uintptr_t w = (uintptr_t)comm->ws;
        for (int r = 0; r < nranks; ++r)
            if (ranges_overlap(w, need, (uintptr_t)sendbufs[r], bytes) ||
                ranges_overlap(w, need, (uintptr_t)recvbufs[r], bytes))
                return reject(arInvalidArgument, "the workspace overlaps a rank buffer");
    }
    if (proto == arProtoLL) {
        if (nranks > comm->max_ranks)
            return reject(arInvalidUsage, "nranks above the communicator's maxRanks");
        if (bytes > comm->max_ll_bytes)
            return reject(arInvalidUsage, "message above the communicator's maxLLBytesPerRank");
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != comm->device)
        return reject(arInvalidUsage, "the communicator's device is not the current device");

    // Launch shape: explicit options, else the tuned shape of this size and
    // mode, else the built-in defaults (0).  A tuned LL entry brings its packet
    // width with it.
    const bool ll = proto == arProtoLL;
    int threads = (int)comm->opt[ll ? arOptLLThreads : arOptHBThreads];
    uint64_t blocks = (uint64_t)comm->opt[ll ? arOptLLBlocksPerRank : arOptHBBlocks];
    int pkt = ll ? (int)comm->opt[arOptLLPacketBytes] : 0;
    // The sequenced LL scheme is an ablation: explicit options or its
    // defaults, never the tuned shape (the tuner times the cleared scheme).
    const int scheme = ll ? (int)comm->opt[arOptLLFlagScheme] : ar::kSchemeCleared;
    // HB access policy: the option if set (0 or 1), else the tuned entry's,
    // else non-temporal.
    int nt = (int)comm->opt[arOptHBNonTemporal];
    const ar::TunedShape &t = comm->tuned[dtype][nranks][proto][in_place][bucket_of(bytes)];
    if (threads == 0 && blocks == 0 && pkt == 0 && scheme == ar::kSchemeCleared &&
        comm->opt[arOptLLDense] < 0 && t.valid) {
        threads = t.threads;
        blocks = (uint64_t)t.blocks;
        pkt = t.pkt_bytes;
        if (nt < 0)
            nt = t.nt;
    }
    if (nt < 0)
        nt = 1;
    // 8-byte packets unless the caller asked for 16 (an ablation: the 16-byte
    // packet relies on each 8-byte half of a 128-bit store becoming visible as
    // a unit, which no document guarantees).
    if (pkt != 16 || !comm->ll16_ok)
        pkt = 8;
    // The staged HB forms take explicit options or their defaults, never the
    // fused kernel's tuned shape.
    const ar::HBConfig cfg = hb_config(comm);
    const int st_threads = (int)comm->opt[arOptHBThreads];
    const uint64_t st_blocks = (uint64_t)comm->opt[arOptHBBlocks];
    const bool st_nt = comm->opt[arOptHBNonTemporal] != 0;
    const hipError_t e =
        two_level ? ar::launch_hb_hier(sendbufs, recvbufs, count, (int)dtype, nranks, group,
                                       comm->ws, cfg, st_threads, st_blocks, st_nt,
                                       (hipStream_t)stream)
        : proto == arProtoHB && staged
            ? ar::launch_hb_staged(sendbufs, recvbufs, count, (int)dtype, nranks, cfg, st_threads,
                                   st_blocks, st_nt, (hipStream_t)stream)
            : launch(sendbufs, recvbufs, count, dtype, nranks, proto, comm, threads, blocks, pkt,
                     scheme, group, nt != 0, (hipStream_t)stream);
    if (e != hipSuccess)
        return reject(arHipError, hipGetErrorString(e));
    return arSuccess;
}

arResult_t arCommTune(arComm_t comm, arDataType_t dtype_arg, int nranks,
                      size_t maxBytesPerRank, arStream_t stream)
{
    if (comm == nullptr)
        return reject(arInvalidArgument, "NULL comm");
    const int dti = raw(dtype_arg);
    if (dti != arBfloat16 && dti != arFloat16 && dti != arFloat32)
        return reject(arUnsupported, "dtype must be bf16, fp16 or fp32");
    const arDataType_t dtype = (arDataType_t)dti;
    if (nranks < 1 || nranks > AR_MAX_RANKS)
        return reject(arUnsupported, "nranks must be in 1..32");
    if (maxBytesPerRank < 512 || maxBytesPerRank > ((size_t)1 << 34))
        return reject(arInvalidArgument, "maxBytesPerRank must be in 512 B .. 16 GiB");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != comm->device)
        return reject(arInvalidUsage, "the communicator's device is not the current device");

    const size_t es = elem_bytes(dtype);
    const size_t stride = (maxBytesPerRank + 255) / 256 * 256;
    const bool fresh = comm->opt[arOptTuneFreshInputs] != 0;
    char *splane = nullptr, *rplane = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipStream_t cs = nullptr;  // private stream: graph capture is not allowed on the null stream
    arResult_t result = arSuccess;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
        hipMalloc((void **)&splane, stride * (size_t)nranks) != hipSuccess ||
        hipMalloc((void **)&rplane, stride * (size_t)nranks) != hipSuccess ||
        hipMemset(splane, 0x3c, stride * (size_t)nranks) != hipSuccess ||
        hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess ||
        hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        result = reject(arHipError, "tuning set-up failed");
    }
    std::vector<const void *> send((size_t)nranks);
    std::vector<void *> recv((size_t)nranks);
    for (int r = 0; r < nranks && result == arSuccess; ++r) {
        send[(size_t)r] = splane + (size_t)r * stride;
        recv[(size_t)r] = rplane + (size_t)r * stride;
    }

    // Candidate shapes: the built-in default first, then a (threads per
    // workgroup, workgroups) grid around it.  The launchers clamp each
    // to what the kernel and the message allow.  A candidate replaces the best
    // so far only if it is more than 3 % faster, so timing noise does not move
    // the choice away from the default.
    static const int kLLThreads[] = {128, 256, 512, 1024};
    static const int kLLBlocks[] = {1, 2, 4, 8, 16, 32, 64};
    static const int kHBThreads[] = {128, 256, 512};

    const int top = bucket_of(maxBytesPerRank);
    for (int b = 9; b <= top && result == arSuccess; ++b) {
        size_t bytes = ((size_t)1 << b) < maxBytesPerRank ? ((size_t)1 << b) : maxBytesPerRank;
        const size_t count = bytes / es > 0 ? bytes / es : 1;
        bytes = count * es;
        // about 200 us of timed work per candidate, between 5 and 20 calls
        // (estimate: each rank's message read and written once at 5 TB/s,
        // plus 3 us)
        const double est_us = (double)(2 * (size_t)nranks * bytes) / 5.0e6 + 3.0;
        int calls = (int)(200.0 / est_us);
        calls = calls < 5 ? 5 : (calls > 20 ? 20 : calls);
        // HB workgroups: half, once and twice the default count for this size
        // (one per CU, or more per CU for few ranks and large messages)
        const int hb_default = comm->cu_count * ar::hb_default_blocks_per_cu(nranks, (uint64_t)bytes);
        const int hb_blocks[] = {hb_default / 2, hb_default, hb_default * 2};
        for (int m = 0; m < 4 && result == arSuccess; ++m) {
            const int proto = m / 2 == 0 ? arProtoLL : arProtoHB;
            const int in_place = m % 2;  // in place: the send plane is also the receive plane
            void *const *dst = in_place ? const_cast<void *const *>(send.data()) : recv.data();
            if (proto == arProtoLL && !ll_possible(comm, nranks, bytes))
                continue;
            // LL: the default shape and the grid, with 8-byte packets (the
            // 16-byte packet is an ablation a caller must ask for).  HB: the
            // same for each access policy (non-temporal first), unless the
            // communicator's option fixes it.
            const int nb = proto == arProtoLL ? 7 : 3;
            const int nth = proto == arProtoLL ? 4 : 3;
            const int per_variant = 1 + nth * nb;
            const int nt_opt = (int)comm->opt[arOptHBNonTemporal];
            const int variants = proto == arProtoLL ? 1 : (nt_opt < 0 ? 2 : 1);
            // Fresh inputs: the rewrites alone are timed first, and each
            // candidate's time is its graph's time less theirs.
            const TuneFill fill = {fresh ? splane : nullptr, stride, bytes / 16, nranks};
            float fill_us = 0.0f;
            if (fresh) {
                const hipError_t e = time_candidate(send.data(), dst, count, dtype, nranks,
                                                    (arProtocol_t)proto, comm, 0, 0, 8,
                                                    ar::kSchemeCleared, true, fill, false, calls,
                                                    cs, e0, e1, &fill_us);
                if (e != hipSuccess) {
                    result = reject(arHipError, hipGetErrorString(e));
                    break;
                }
            }
            ar::TunedShape best = {0, 0, 0, 0, 0, 0.0f};
            for (int cw = 0; cw < variants * per_variant && result == arSuccess; ++cw) {
                const int c = cw % per_variant - 1;
                const int var = cw / per_variant;
                const int pkt = proto == arProtoLL ? 8 : 0;
                const int nt = proto == arProtoLL ? 0 : (nt_opt >= 0 ? nt_opt : (var == 0 ? 1 : 0));
                const int th = c < 0 ? 0 : (proto == arProtoLL ? kLLThreads[c / nb] : kHBThreads[c / nb]);
                const int bl = c < 0 ? 0 : (proto == arProtoLL ? kLLBlocks[c % nb] : hb_blocks[c % nb]);
                float us = 0.0f;
                const hipError_t e = time_candidate(send.data(), dst, count, dtype, nranks,
                                                    (arProtocol_t)proto, comm, th, (uint64_t)bl,
                                                    pkt, ar::kSchemeCleared, nt != 0, fill, true,
                                                    calls, cs, e0, e1, &us);
                if (e != hipSuccess) {
                    result = reject(arHipError, hipGetErrorString(e));
                    break;
                }
                // (a difference, so timing noise can take it to zero or below)
                us = fresh ? (us - fill_us > 0.01f ? us - fill_us : 0.01f) : us;
                if (!best.valid || us < 0.97f * best.us)
                    best = {1, th, bl, pkt, nt, us};
            }
            // A winner other than the built-in default is timed once more beside
            // the default and kept only if it still wins by 3 %: single timings
            // at these sizes scatter by several percent (at 16 ranks and 1 MiB
            // per rank a shape that had won that way ran 9 % slower than the
            // default in use).
            const int def_nt = proto == arProtoLL ? 0 : (nt_opt >= 0 ? nt_opt : 1);
            if (result == arSuccess && best.valid &&
                (best.threads != 0 || best.blocks != 0 || best.nt != def_nt)) {
                float d_us = 0.0f, w_us = 0.0f;
                hipError_t e = time_candidate(send.data(), dst, count, dtype, nranks,
                                              (arProtocol_t)proto, comm, 0, 0, best.pkt_bytes,
                                              ar::kSchemeCleared, def_nt != 0, fill, true, calls,
                                              cs, e0, e1, &d_us);
                if (e == hipSuccess)
                    e = time_candidate(send.data(), dst, count, dtype, nranks,
                                       (arProtocol_t)proto, comm, best.threads,
                                       (uint64_t)best.blocks, best.pkt_bytes, ar::kSchemeCleared,
                                       best.nt != 0, fill, true, calls, cs, e0, e1, &w_us);
                if (e != hipSuccess) {
                    result = reject(arHipError, hipGetErrorString(e));
                } else {
                    if (fresh) {
                        d_us = d_us - fill_us > 0.01f ? d_us - fill_us : 0.01f;
                        w_us = w_us - fill_us > 0.01f ? w_us - fill_us : 0.01f;
                    }
                    if (!(w_us < 0.97f * d_us))
                        best = {1, 0, 0, best.pkt_bytes, def_nt, d_us};
                }
            }
            if (result == arSuccess)
                comm->tuned[dtype][nranks][proto][in_place][b] = best;
        }
    }
    if (e0 != nullptr)
        (void)hipEventDestroy(e0);
    if (e1 != nullptr)
        (void)hipEventDestroy(e1);
    if (hipDeviceSynchronize() != hipSuccess && result == arSuccess)
        result = reject(arHipError, "synchronisation after tuning failed");
    if (cs != nullptr)
        (void)hipStreamDestroy(cs);
    (void)hipFree(splane);
    (void)hipFree(rplane);
    if (result == arSuccess) {
        uint32_t word = 0;
        if (hipMemcpy(&word, comm->ctrl + 0, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
            result = reject(arHipError, "reading the error word failed");
        else if (word != 0)
            result = reject(arTimeout, "an LL wait timed out while tuning");
    }
    return result;
}

arResult_t arAllReduceNoAlloc(const void *const *sendbufs, void *const *recvbufs, size_t count,
                              arDataType_t dtype_arg, arRedOp_t op_arg, int nranks,
                              int nodeRanks, arStream_t stream)
{
    arResult_t r = validate(sendbufs, recvbufs, count, raw(dtype_arg), raw(op_arg), nranks,
                            arProtoHB);
    if (r != arSuccess)
        return r;
    if (nodeRanks < 0 || nodeRanks > AR_MAX_RANKS)
        return reject(arInvalidArgument, "nodeRanks must be in 0..32");
    if (count == 0)
        return arSuccess;
    const int group = nodeRanks > 1 && nodeRanks < nranks ? nodeRanks : 0;
    if (group != 0 && nranks % group != 0)
        return reject(arInvalidUsage, "nranks is not a multiple of nodeRanks");
    if (group != 0 &&
        ar::hier_workspace_bytes(count, nranks / group) > (uint64_t)AR_NOALLOC_SCRATCH_BYTES)
        return reject(arInvalidUsage, "the node partials exceed AR_NOALLOC_SCRATCH_BYTES");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices)
        return reject(arHipError, "no usable current device");
    NoAllocDevice d = {};
    r = noalloc_device(dev, &d);
    if (r != arSuccess)
        return r;
    // Each kernel's default launch shape (as arAllReduce with no shape
    // options), non-temporal accesses, interleaved chunks; no launch record.
    const ar::HBConfig cfg = {d.cu_count, 1, true, nullptr};
    const int dtype = raw(dtype_arg);
    const hipError_t e =
        group != 0 ? ar::launch_hb_hier(sendbufs, recvbufs, count, dtype, nranks, group, d.scratch,
                                        cfg, 0, 0, true, (hipStream_t)stream)
                   : ar::launch_hb(sendbufs, recvbufs, count, dtype, nranks, cfg, 0, 0, 0, true,
                                   (hipStream_t)stream);
    if (e != hipSuccess)
        return reject(arHipError, hipGetErrorString(e));
    return arSuccess;
}

arResult_t arCommGetLastLaunch(arComm_t comm, arLaunchInfo_t *info)
{
    if (comm == nullptr || info == nullptr)
        return reject(arInvalidArgument, "NULL argument");
    const ar::LaunchRecord &l = comm->last;
    info->protocol = l.protocol;
    info->kernels = l.kernels;
    info->grid = l.grid;
    info->threads = l.threads;
    info->packetBytes = l.pkt_bytes;
    info->packetPayloadBytes = l.payload;
    info->nonTemporal = l.nt;
    info->nodeRanks = l.node;
    info->staged = l.staged;
    return arSuccess;
}

arResult_t arCommGetTunedShape(arComm_t comm, arDataType_t dtype_arg, int nranks,
                               arProtocol_t protocol_arg, size_t bytesPerRank, int inPlace,
                               arTunedShape_t *shape)
{
    if (comm == nullptr || shape == nullptr)
        return reject(arInvalidArgument, "NULL argument");
    const int dtype = raw(dtype_arg), protocol = raw(protocol_arg);
    if ((dtype != arBfloat16 && dtype != arFloat16 && dtype != arFloat32) || nranks < 1 ||
        nranks > AR_MAX_RANKS || (protocol != arProtoLL && protocol != arProtoHB) ||
        bytesPerRank == 0 || (inPlace != 0 && inPlace != 1))
        return reject(arInvalidArgument, "argument out of range");
    const ar::TunedShape &t =
        comm->tuned[dtype][nranks][protocol][inPlace][bucket_of(bytesPerRank)];
    shape->tuned = t.valid;
    shape->threads = t.threads;
    shape->blocks = t.blocks;
    shape->packetBytes = t.pkt_bytes;
    shape->nonTemporal = t.nt;
    shape->us = t.us;
    return arSuccess;
}

}  // extern "C"
