// ll_oneshot.hip -- the low-latency (LL) all-reduce: one shot, flagged packets.
//
// The LL protocol of the MemoryChannel table in "MSCCL++：让 GPU 通信像 CUDA
// 一样可编程" (infinitensor.com/news/50) trades bandwidth for frequent,
// fine-grained synchronisation, for decode-size messages.  Its device-side
// building blocks are a one-sided put of data plus a signal, and a wait on the
// other side (the microsoft/mscclpp project summary, agentlenshq.com, "How it
// works": put/signal/wait with no matching receive).  Here put and signal are
// one 64-bit store: a 4-byte payload next to a 4-byte flag, so a reader that
// sees the flag also sees the payload, with no separate fence or counter.
//
// One kernel does the whole call for all R simulated ranks.  Workgroup
// w = b * R + k acts for rank k on slice b of the message:
//   put     rank k's words of slice b become packets {payload, ready} in rank
//           k's packet region (the stand-in for peer memory);
//   poll    the workgroup takes sub-slice k of slice b and, lane by lane,
//           re-reads the R packets of each word until all R are ready --
//           R - 1 of them are written by other workgroups, which for R = 8
//           sit on the other seven XCDs;
//   reduce  binary32 sum in rank order 0..R-1, rounded once to the dtype;
//   clear   the R packets go back to zero;
//   output  the word goes to all R receive buffers.
// In place is safe: a word is written out only after all R packets for it
// arrived, and each packet carries a value its producer had already read.
//
// Packet memory is all zero between calls: every packet a call writes is
// consumed and cleared by the same call, and the next call (on the same
// stream, or the next node of a replayed graph) starts after this kernel has
// ended.  So a packet is ready exactly when its flag is nonzero, and no
// per-call sequence number is needed.  That keeps graph replays correct with
// frozen kernel arguments and needs no shared counter: a device-wide counter
// bumped once per workgroup costs a serialised atomic per workgroup on one
// address, which measured about 15 ns each on MI355X (5 us for the 512
// workgroups of a 1 MiB-per-rank call).
// A wait is bounded by a wall-clock limit: on expiry the lane records
// arTimeout in the communicator and stops waiting.  Packets of an interrupted
// call may then stay set, so after arTimeout the communicator must be reset
// (arCommReset) before further LL calls.  Every workgroup of the grid must be
// resident at once (the host caps the grid with the occupancy calculator),
// because consumers wait on producers.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

// Largest workgroup compiled for a rank-table size (the polled packets of a
// lane, 2 VGPRs each, must fit the register share of that many threads).
constexpr int ll_max_threads(int rmax) { return rmax >= 32 ? 512 : 1024; }
// Words a lane polls at once: R packets each, all loads in flight together.
constexpr int ll_get_batch(int rmax) { return rmax <= 8 ? 2 : 1; }
// Source words a lane loads before it stores their packets.
constexpr int kPutBatch = 8;
// Flag of a ready packet; cleared packet memory reads 0.
constexpr uint32_t kReady = 1u;

template <typename T, int RMAX, bool EXACT>
__global__ __launch_bounds__(ll_max_threads(RMAX)) void ll_oneshot(LLParams<RMAX> p)
{
    constexpr int GB = ll_get_batch(RMAX);
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint32_t nthr = blockDim.x;
    const uint32_t k = blockIdx.x % n;
    const uint32_t b = blockIdx.x / n;

    // put: publish rank k's words of slice b
    const uint64_t p0 = (uint64_t)b * p.put_per_block;
    const uint64_t p1 = (p0 + p.put_per_block < p.npkt) ? p0 + p.put_per_block : p.npkt;
    const uint32_t *src = (const uint32_t *)p.rk.send[k];
    uint64_t *mine = p.pkts + (uint64_t)k * p.pkt_stride;
    // Whole 4-byte words go through the batches; a message of odd 16-bit
    // length ends in one 2-byte word, handled by a single lane below.
    const uint64_t nfull = p.npkt - p.half_tail;
    const uint64_t pf = p1 < nfull ? p1 : nfull;
    const uint64_t pstep = (uint64_t)kPutBatch * nthr;
    for (uint64_t pbase = p0 + threadIdx.x; pbase < pf; pbase += pstep) {
        uint32_t w[kPutBatch];
#pragma unroll
        for (int v = 0; v < kPutBatch; ++v) {
            const uint64_t q = pbase + (uint64_t)v * nthr;
            if (q < pf)
                w[v] = src[q];
        }
        // gfx9 counts loads and stores on one counter that runs out of order
        // once both are pending, so a load result needed after a store forces
        // a wait for everything.  One explicit wait for the batch's loads
        // lets its stores issue back to back.
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int v = 0; v < kPutBatch; ++v) {
            const uint64_t q = pbase + (uint64_t)v * nthr;
            if (q < pf)
                put_packet(mine + q, w[v], kReady);
        }
    }
    if (p.half_tail && threadIdx.x == 0 && nfull >= p0 && nfull < p1)
        put_packet(mine + nfull, (uint32_t)((const uint16_t *)(src + nfull))[0], kReady);

    // poll, reduce, clear, output: sub-slice k of slice b
    const uint32_t want = kReady + p.flag_skew;
    const uint64_t g0 = p0 + (uint64_t)k * p.get_per_block;
    const uint64_t g1 = (g0 + p.get_per_block < p1) ? g0 + p.get_per_block : p1;
    // Two bounds on a lane's total waiting: wall-clock ticks (10 ns each at
    // the 100 MHz real-time clock), and, in case the clock were to stall, a
    // re-read count: a device-scope load takes well over 100 ns, so as many
    // re-reads as ticks outlast the wall-clock bound about tenfold.
    uint64_t wait_start = 0;
    uint64_t spins = 0;
    const uint64_t spin_limit = p.timeout_ticks;
    bool gave_up = false;
    for (uint64_t q0 = g0 + threadIdx.x; q0 < g1 && !gave_up; q0 += (uint64_t)GB * nthr) {
        uint64_t pk[GB][RMAX];
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = q0 + (uint64_t)v * nthr;
            if (q < g1) {
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    if (EXACT || j < (int)n)
                        pk[v][j] = read_packet(p.pkts + (uint64_t)j * p.pkt_stride + q);
            }
        }
        for (;;) {
            bool ready = true;
#pragma unroll
            for (int v = 0; v < GB; ++v)
                if (q0 + (uint64_t)v * nthr < g1)
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if (EXACT || j < (int)n)
                            ready = ready && packet_flag(pk[v][j]) == want;
            if (ready)
                break;
            const uint64_t now = wall_clock64();
            if (wait_start == 0)
                wait_start = now;
            else if (now - wait_start > p.timeout_ticks || ++spins > spin_limit) {
                __hip_atomic_store(p.ctrl + 0, (uint32_t)arTimeout, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                gave_up = true;
                break;
            }
#pragma unroll
            for (int v = 0; v < GB; ++v) {
                const uint64_t q = q0 + (uint64_t)v * nthr;
                if (q < g1) {
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if ((EXACT || j < (int)n) && packet_flag(pk[v][j]) != want)
                            pk[v][j] = read_packet(p.pkts + (uint64_t)j * p.pkt_stride + q);
                }
            }
        }
        if (gave_up)
            break;

#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = q0 + (uint64_t)v * nthr;
            if (q >= g1)
                continue;
            float acc[T::kPerWord];
            T::widen(packet_payload(pk[v][0]), acc);
#pragma unroll
            for (int j = 1; j < RMAX; ++j) {
                if (EXACT || j < (int)n) {
                    float x[T::kPerWord];
                    T::widen(packet_payload(pk[v][j]), x);
#pragma unroll
                    for (int e = 0; e < T::kPerWord; ++e)
                        acc[e] = acc[e] + x[e];
                }
            }
            const uint32_t y = T::narrow(acc);
#pragma unroll
            for (int j = 0; j < RMAX; ++j)
                if (EXACT || j < (int)n)
                    put_packet(p.pkts + (uint64_t)j * p.pkt_stride + q, 0u, 0u);
            const bool half = p.half_tail && q == p.npkt - 1;
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (EXACT || r < (int)n) {
                    uint32_t *dst = (uint32_t *)p.rk.recv[r] + q;
                    if (half)
                        *(uint16_t *)dst = (uint16_t)y;
                    else
                        *dst = y;
                }
            }
        }
    }
}

// Clears the async-error word and all packets (vector stores; no memset node
// in graphs).
__global__ __launch_bounds__(256) void ll_reset(uint64_t *pkts, uint64_t npkts, uint32_t *ctrl)
{
    const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = i0; i < npkts; i += step)
        pkts[i] = 0;
    if (i0 < 16)
        ctrl[i0] = 0;
}

namespace {

constexpr int kThreadOptions[kThreadChoices] = {64, 128, 256, 512, 1024};

int thread_index(int threads)
{
    for (int i = 0; i < kThreadChoices; ++i)
        if (kThreadOptions[i] == threads)
            return i;
    return 2;
}

// rank-table variant index: 0..5 exact {1,2,4,8,16,32}; 6 generic (any)
int variant_of(int nranks)
{
    switch (nranks) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    case 16: return 4;
    case 32: return 5;
    default: return 6;
    }
}

template <typename T, int RMAX, bool EXACT>
hipError_t launch_table(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int want_threads, uint64_t want_blocks,
                        hipStream_t stream)
{
    LLParams<RMAX> p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    const uint64_t bytes = (uint64_t)count * T::kBytes;
    p.npkt = (bytes + 3) / 4;
    p.half_tail = (bytes % 4) != 0;
    p.pkts = comm->pkts;
    p.pkt_stride = comm->pkt_stride;
    p.ctrl = comm->ctrl;
    p.nranks = (uint32_t)nranks;
    p.flag_skew = (uint32_t)comm->opt[arOptDebugFlagSkew];
    p.timeout_ticks = (uint64_t)comm->opt[arOptPollTimeoutUs] * comm->wall_clock_khz / 1000u;

    // Default launch shape, measured on MI355X for R = 8 bf16 from 2 KiB to
    // 1 MiB per rank: 256-thread workgroups (512 from 512 KiB per rank up),
    // about two words per lane, at most 64 workgroups per rank (32 from
    // 256 KiB per rank up).
    int threads = want_threads;
    if (threads <= 0)
        threads = p.npkt >= 131072 ? 512 : 256;
    if (threads > ll_max_threads(RMAX))
        threads = ll_max_threads(RMAX);
    const int resident = comm->ll_resident[T::kId][variant_of(nranks)][thread_index(threads)];
    uint64_t max_per_rank = (uint64_t)(resident / nranks);
    if (max_per_rank < 1)
        max_per_rank = 1;

    uint64_t per_rank = want_blocks;
    if (per_rank == 0) {
        const uint64_t cap = p.npkt >= 65536 ? 32 : 64;
        per_rank = (p.npkt + (uint64_t)threads * 2 - 1) / ((uint64_t)threads * 2);
        if (per_rank > cap)
            per_rank = cap;
    }
    if (per_rank > max_per_rank)
        per_rank = max_per_rank;
    if (per_rank > p.npkt)
        per_rank = p.npkt;
    if (per_rank < 1)
        per_rank = 1;
    p.put_per_block = (p.npkt + per_rank - 1) / per_rank;
    p.get_per_block = (p.put_per_block + (uint64_t)nranks - 1) / (uint64_t)nranks;
    p.blocks_per_rank = (uint32_t)per_rank;
    const uint32_t grid = (uint32_t)(per_rank * (uint64_t)nranks);

    hipLaunchKernelGGL((ll_oneshot<T, RMAX, EXACT>), dim3(grid), dim3(threads), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int th, uint64_t bl, hipStream_t stream)
{
    switch (nranks) {
    case 1: return launch_table<T, 1, true>(send, recv, count, nranks, comm, th, bl, stream);
    case 2: return launch_table<T, 2, true>(send, recv, count, nranks, comm, th, bl, stream);
    case 4: return launch_table<T, 4, true>(send, recv, count, nranks, comm, th, bl, stream);
    case 8: return launch_table<T, 8, true>(send, recv, count, nranks, comm, th, bl, stream);
    case 16: return launch_table<T, 16, true>(send, recv, count, nranks, comm, th, bl, stream);
    case 32: return launch_table<T, 32, true>(send, recv, count, nranks, comm, th, bl, stream);
    default: return launch_table<T, 32, false>(send, recv, count, nranks, comm, th, bl, stream);
    }
}

template <typename T, int RMAX, bool EXACT>
hipError_t query_one(int *out)
{
    for (int i = 0; i < kThreadChoices; ++i) {
        if (kThreadOptions[i] > ll_max_threads(RMAX)) {
            out[i] = 0;  // never launched with this many threads
            continue;
        }
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&ll_oneshot<T, RMAX, EXACT>),
            kThreadOptions[i], 0);
        if (e != hipSuccess)
            return e;
        out[i] = per_cu;
    }
    return hipSuccess;
}

template <typename T>
hipError_t query_dtype(int (*tab)[kThreadChoices])
{
    hipError_t e;
    if ((e = query_one<T, 1, true>(tab[0])) != hipSuccess) return e;
    if ((e = query_one<T, 2, true>(tab[1])) != hipSuccess) return e;
    if ((e = query_one<T, 4, true>(tab[2])) != hipSuccess) return e;
    if ((e = query_one<T, 8, true>(tab[3])) != hipSuccess) return e;
    if ((e = query_one<T, 16, true>(tab[4])) != hipSuccess) return e;
    if ((e = query_one<T, 32, true>(tab[5])) != hipSuccess) return e;
    return query_one<T, 32, false>(tab[6]);
}

}  // namespace

hipError_t launch_ll(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const arComm *comm, int threads, uint64_t blocks,
                     hipStream_t stream)
{
    switch (dtype) {
    case kBf16: return launch_dtype<Bf16>(send, recv, count, nranks, comm, threads, blocks, stream);
    case kFp16: return launch_dtype<Fp16>(send, recv, count, nranks, comm, threads, blocks, stream);
    default: return launch_dtype<Fp32>(send, recv, count, nranks, comm, threads, blocks, stream);
    }
}

hipError_t launch_reset(const arComm *comm, hipStream_t stream)
{
    const uint64_t npkts = (uint64_t)comm->max_ranks * comm->pkt_stride;
    uint64_t blocks = (npkts + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(ll_reset, dim3((uint32_t)blocks), dim3(256), 0, stream, comm->pkts, npkts,
                       comm->ctrl);
    return hipGetLastError();
}

hipError_t query_ll_residency(arComm *comm)
{
    int per_cu[3][kRankVariants + 1][kThreadChoices] = {};
    hipError_t e;
    if ((e = query_dtype<Bf16>(per_cu[kBf16])) != hipSuccess) return e;
    if ((e = query_dtype<Fp16>(per_cu[kFp16])) != hipSuccess) return e;
    if ((e = query_dtype<Fp32>(per_cu[kFp32])) != hipSuccess) return e;
    for (int d = 0; d < 3; ++d)
        for (int v = 0; v <= kRankVariants; ++v)
            for (int t = 0; t < kThreadChoices; ++t)
                comm->ll_resident[d][v][t] = per_cu[d][v][t] * comm->cu_count;
    return hipSuccess;
}

}  // namespace ar
