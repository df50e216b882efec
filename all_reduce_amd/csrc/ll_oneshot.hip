// ll_oneshot.hip -- the low-latency (LL) all-reduce: one shot, flagged packets.
//
// The LL protocol of the MemoryChannel table in "MSCCL++：让 GPU 通信像 CUDA
// 一样可编程" (infinitensor.com/news/50) trades bandwidth for frequent,
// fine-grained synchronisation, for decode-size messages.  Its device-side
// building blocks are a one-sided put of data plus a signal, and a wait on the
// other side (the microsoft/mscclpp project summary, agentlenshq.com, "How it
// works": put/signal/wait with no matching receive).  Here put and signal are
// one store: a 4-byte payload next to a 4-byte flag (an 8-byte packet), or two
// such pairs in one 16-byte packet, so a reader that sees the flags also sees
// the payload, with no separate fence or counter.
//
// One kernel does the whole call for all R simulated ranks.  Workgroup
// w = b * R + k acts for rank k on slice b of the message:
//   put     rank k's words of slice b become packets {payload, ready} in rank
//           k's packet region (the stand-in for peer memory);
//   poll    the workgroup takes sub-slice k of slice b and, lane by lane,
//           re-reads the R packets of each packet index until all R are ready --
//           R - 1 of them are written by other workgroups, which for R = 8
//           sit on the other seven XCDs;
//   reduce  binary32 sum in rank order 0..R-1, rounded once to the dtype;
//   retire  the R packets are made unable to look ready to a later call;
//   output  the word goes to all R receive buffers.
// In place is safe: a word is written out only after all R packets for it
// arrived, and each packet carries a value its producer had already read.
//
// A reader must never take a packet left by an earlier call for a new one.
// Kernel arguments are frozen in a replayed graph, so the flag value cannot
// come from the host, and a device-wide call counter would need a serialised
// atomic per workgroup on one address to advance safely (about 15 ns each on
// MI355X, 5 us for the 512 workgroups of a 1 MiB-per-rank call).  Two flag
// schemes avoid both:
//
//   cleared    (SEQ = false) the reader zeroes every packet it has consumed,
//              so packet memory is zero between calls and a packet is ready
//              when its flag holds the constant kReady.  Costs one store per
//              packet: a quarter of the scheme's memory traffic.
//   sequenced  (SEQ = true) every 512-byte group of a rank's packet region has
//              a 32-bit sequence number in a side table.  Producers write the
//              group's next number as the flag; the one wave that consumes
//              the group (the launch aligns every wave's packets to whole
//              groups) waits for it, then advances the table entry.  Between
//              calls every nonzero packet of a group carries the entry's
//              current number, so the next number cannot be mistaken for a
//              stale one, even after the 32-bit count wraps.  Nothing is
//              cleared except the packets past the end of the message in its
//              last group (fewer than 64 per rank).  Every producer reads the
//              entry before it stores the packets the consumer waits for, so
//              all reads of an entry precede its update.
//
// The schemes interleave freely on one communicator: kReady is a value the
// sequenced scheme never writes, and a cleared call leaves zeros.  The cleared
// scheme is the default: on MI355X it is faster at every LL size.  Hardware
// counters on both (R = 8 bf16, 256 KiB to 1 MiB per rank) show why: the
// sequenced scheme writes 40% fewer bytes, but every 512-byte group costs one
// table read on each side -- as many extra vector memory reads as the cleared
// scheme issues in all -- and both sit on the critical path, before a
// producer's first store and before a consumer's first poll, whereas the
// clears the table saves are stores no one waits for.
// A wait is bounded by a wall-clock limit: on expiry the lane records
// arTimeout in the communicator and stops waiting.  Packets of an interrupted
// call may then stay set and table entries stay behind, so after arTimeout
// the communicator must be reset (arCommReset) before further LL calls.
// Every workgroup of the grid must be resident at once (the host caps the
// grid with the occupancy calculator), because consumers wait on producers.
#include "ar_internal.hpp"
#include "ll_packet.hpp"

namespace ar {

// One-shot LL launch parameters.
template <int R>
struct LLParams {
    RankTable<R> rk;
    uint64_t *pkts;          // packet scratch; rank k's packets start at k * pkt_stride
    uint64_t pkt_stride;     // packets of this launch's width per rank region
    uint64_t region_bytes;   // size of the whole packet scratch
    uint64_t npkt;           // packets per rank = ceil(bytes per rank / payload bytes)
    uint64_t put_per_block;  // packets each workgroup publishes for its rank
    uint64_t get_per_block;  // packets each workgroup polls, reduces and writes out
    uint32_t *ctrl;          // [0] async error (0 or arTimeout)
    uint32_t *seq;           // sequenced scheme: entry of 512-byte group g, rank j at g * seq_stride + j
    uint64_t seq_stride;
    uint64_t timeout_ticks;  // wall-clock ticks one packet wait may take
    uint32_t flag_skew;      // test hook: consumers wait for flag + skew
    uint32_t tail_bytes;     // payload bytes of a last, partial packet (0: none)
    uint32_t nranks;
    uint32_t blocks_per_rank;
    uint32_t node_starts;    // bitmask node layout: bit j set where rank j starts a node, j > 0
};

// Largest workgroup compiled for a rank-table size (the polled packets of a
// lane, 2 or 4 VGPRs each, must fit the register share of that many threads).
constexpr int ll_max_threads(int rmax) { return rmax >= 32 ? 512 : 1024; }
// Packets a lane polls at once: R packets each, all loads in flight together
// (the same bytes in flight for both widths).
constexpr int ll_get_batch(int rmax, int pw) { return rmax * pw <= 8 ? 2 : 1; }
// Source packets' worth of words a lane loads before it stores their packets.
constexpr int kPutBatch = 8;
// Flag of a ready packet in the cleared scheme; cleared packet memory reads 0,
// and the sequenced scheme never writes this value.
constexpr uint32_t kReady = 0xffffffffu;
// Packets in one 512-byte group of the sequenced scheme.
constexpr uint64_t seq_group(int pw) { return 64 / pw; }

// The sequence number after s: never 0 (fresh memory) nor kReady.
__device__ inline uint32_t next_seq(uint32_t s) { return s >= 0xfffffffeu ? 1u : s + 1u; }

// Table entries are read at agent scope, like the packets, and written with
// ordinary stores: within a call nothing reads an entry after its update (see
// above), and the kernel boundary makes the writes visible to the next call.
__device__ inline uint32_t load_seq(const uint32_t *e)
{
    return __hip_atomic_load(const_cast<uint32_t *>(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void store_seq(uint32_t *e, uint32_t v)
{
    __hip_atomic_store(e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// PW: payload words per packet (1: 8-byte packets; 2: 16-byte packets).
// SEQ: the sequenced flag scheme, else the cleared one.
// NODE: kNodeFlat for the flat order, else the hierarchical order -- the
// ranks form nodes of consecutive ranks, each node's partial is summed in
// binary32 in rank order, then the partials in node order, then one rounding.
// Nodes of NODE ranks when NODE > 0, which makes every node boundary a
// compile-time fact of the unrolled rank loop; with kNodeMask, p.node_starts
// marks where each node after the first begins, a per-rank select that costs
// a second addition and two selects per value (on MI355X, 16-byte packets at
// 32 ranks ran 10-18 % slower with the mask than in the flat order).
template <typename T, int RMAX, bool EXACT, int PW, bool SEQ, int NODE = kNodeFlat>
__global__ __launch_bounds__(ll_max_threads(RMAX)) void ll_oneshot(LLParams<RMAX> p)
{
    constexpr int GB = ll_get_batch(RMAX, PW);
    constexpr uint64_t G = seq_group(PW);
    using IO = PacketIO<PW>;
    using V = typename IO::V;
    const IO io(p.pkts, p.region_bytes);
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint32_t nthr = blockDim.x;
    const uint32_t k = blockIdx.x % n;
    const uint32_t b = blockIdx.x / n;
    // Generic tables (a rank count without its own kernel): the output
    // pointers come from a wave-held copy (WaveTable), and the run-time count
    // is re-read each round below; hoisted, the per-rank tests and pointers
    // spill out of scalar registers.  On MI355X, bf16 at 2 KiB per rank:
    // 12 ranks 4.7 against 5.3 us, 24 ranks 7.3 against 9.0 us.  The exact
    // tables keep the scalar one (16 and 32 ranks: 3-8 % faster).
    constexpr bool kWT = !EXACT;
    WaveTable<RMAX> wt;
    if constexpr (kWT)
        wt = WaveTable<RMAX>(p.rk);

    // put: publish rank k's packets of slice b
    const uint64_t p0 = (uint64_t)b * p.put_per_block;
    const uint64_t p1 = (p0 + p.put_per_block < p.npkt) ? p0 + p.put_per_block : p.npkt;
    const uint32_t *src = (const uint32_t *)p.rk.send[k];
    const uint64_t mine = (uint64_t)k * p.pkt_stride;
    // Whole packets go through the batches; a message that ends inside a
    // packet (2, 4 or 6 bytes of it) has that last packet handled by a single
    // lane below.
    const uint64_t nfull = p.npkt - (p.tail_bytes != 0 ? 1 : 0);
    const uint64_t pf = p1 < nfull ? p1 : nfull;
    const uint64_t pstep = (uint64_t)kPutBatch * nthr;
    for (uint64_t pbase = p0 + threadIdx.x; pbase < pf; pbase += pstep) {
        uint32_t w[kPutBatch][PW];
        uint32_t sq[kPutBatch];
#pragma unroll
        for (int v = 0; v < kPutBatch; ++v) {
            const uint64_t q = pbase + (uint64_t)v * nthr;
            if (q < pf) {
                if constexpr (SEQ)
                    sq[v] = load_seq(p.seq + (q / G) * p.seq_stride + k);
                if constexpr (PW == 1) {
                    w[v][0] = src[q];
                } else {
                    const uint2 x = ((const uint2 *)src)[q];
                    w[v][0] = x.x;
                    w[v][1] = x.y;
                }
            }
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
                io.store(mine + q, w[v], SEQ ? next_seq(sq[v]) : kReady);
        }
    }
    if (p.tail_bytes != 0 && threadIdx.x == 0 && nfull >= p0 && nfull < p1) {
        // 2 bytes (8-byte packets), or 2, 4 or 6 bytes (16-byte packets)
        uint32_t w[PW] = {};
        const uint32_t *t = src + nfull * PW;
        const bool word = PW == 2 && p.tail_bytes >= 4;
        if (word)
            w[0] = t[0];
        if (p.tail_bytes & 2u)
            w[word ? 1 : 0] = ((const uint16_t *)t)[word ? 2 : 0];
        const uint32_t f =
            SEQ ? next_seq(load_seq(p.seq + (nfull / G) * p.seq_stride + k)) : kReady;
        io.store(mine + nfull, w, f);
    }

    // Sequenced scheme: packets past the message's end in its last group go
    // back to zero, so that every nonzero packet of a group carries the
    // group's entry once the entry advances.  No reader touches them.
    if constexpr (SEQ) {
        const uint64_t extra = (G - p.npkt % G) % G;
        if (extra != 0 && blockIdx.x == gridDim.x - 1) {
            for (uint32_t t = threadIdx.x; t < extra * n; t += nthr)
                io.clear((uint64_t)(t / extra) * p.pkt_stride + p.npkt + t % extra);
        }
    }

    // poll, reduce, retire, output: sub-slice k of slice b
    // (the debug skew makes the wanted flag one that no producer writes)
    const uint32_t want_cleared = kReady - p.flag_skew;
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
        // With the wave-held table the run-time rank count is re-read each
        // round too: hoisted, the per-rank tests it feeds would hold scalar
        // registers across the loop.
        uint32_t nl = n;
        if constexpr (kWT) {
            wt.refresh();
            if constexpr (!EXACT)
                asm volatile("" : "+s"(nl));
        }
        V pk[GB][RMAX];
        uint32_t sq[SEQ ? GB : 1][SEQ ? RMAX : 1];  // sequenced: the groups' next numbers
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = q0 + (uint64_t)v * nthr;
            if (q < g1) {
                if constexpr (SEQ) {
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if (EXACT || j < (int)nl)
                            sq[v][j] = load_seq(p.seq + (q / G) * p.seq_stride + j);
                }
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    if (EXACT || j < (int)nl)
                        pk[v][j] = io.load((uint64_t)j * p.pkt_stride + q);
            }
        }
        if constexpr (SEQ) {
#pragma unroll
            for (int v = 0; v < GB; ++v)
                if (q0 + (uint64_t)v * nthr < g1)
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if (EXACT || j < (int)nl)
                            sq[v][j] = next_seq(sq[v][j]);
        }
        for (;;) {
            bool ready = true;
#pragma unroll
            for (int v = 0; v < GB; ++v)
                if (q0 + (uint64_t)v * nthr < g1)
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if (EXACT || j < (int)nl)
                            ready = ready && IO::ready(pk[v][j], SEQ ? sq[v][j] + p.flag_skew
                                                                     : want_cleared);
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
                        if ((EXACT || j < (int)nl) &&
                            !IO::ready(pk[v][j], SEQ ? sq[v][j] + p.flag_skew : want_cleared))
                            pk[v][j] = io.load((uint64_t)j * p.pkt_stride + q);
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
            uint32_t y[PW];
#pragma unroll
            for (int e = 0; e < PW; ++e) {
                float acc[T::kPerWord];
                // The running total of finished nodes starts at -0, which
                // leaves the first partial added to it exactly as it is
                // (x + -0 is x for every binary32 x, signed zeros included).
                float total[T::kPerWord];
#pragma unroll
                for (int i = 0; i < T::kPerWord; ++i)
                    total[i] = -0.0f;
                T::widen(IO::word(pk[v][0], e), acc);
#pragma unroll
                for (int j = 1; j < RMAX; ++j) {
                    if (EXACT || j < (int)nl) {
                        float x[T::kPerWord];
                        T::widen(IO::word(pk[v][j], e), x);
                        bool starts_node = false;
                        if constexpr (NODE > 0)
                            starts_node = j % NODE == 0;
                        else if constexpr (NODE == kNodeMask)
                            starts_node = (p.node_starts >> j) & 1u;
                        if (starts_node) {
                            // a node is complete: fold its partial in
#pragma unroll
                            for (int i = 0; i < T::kPerWord; ++i) {
                                total[i] = total[i] + acc[i];
                                acc[i] = x[i];
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < T::kPerWord; ++i)
                                acc[i] = acc[i] + x[i];
                        }
                    }
                }
                if constexpr (NODE != kNodeFlat) {
#pragma unroll
                    for (int i = 0; i < T::kPerWord; ++i)
                        acc[i] = total[i] + acc[i];
                }
                y[e] = T::narrow(acc);
            }
            if constexpr (SEQ) {
                // The whole wave has seen its groups' packets (the poll loop
                // reconverges first); the lane at a group's first packet
                // advances the group's entries.
                if (q % G == 0) {
#pragma unroll
                    for (int j = 0; j < RMAX; ++j)
                        if (EXACT || j < (int)nl)
                            store_seq(p.seq + (q / G) * p.seq_stride + j, sq[v][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    if (EXACT || j < (int)nl)
                        io.clear((uint64_t)j * p.pkt_stride + q);
            }
            // Whole words go out at agent scope, written through to memory:
            // on MI355X that measured 2-4 % faster than write-back stores from
            // 32 KiB per rank up (the same as the packets, whose clears must
            // be written through too), and the outputs are not read here.
            // The message's last, partial packet is tested once per word, not
            // once per rank inside the unrolled store loop: one branch instead
            // of R (2-8 % faster at 2-64 KiB per rank, most at 32 ranks).
            const bool partial = p.tail_bytes != 0 && q == p.npkt - 1;
            if (!partial) {
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    if (EXACT || r < (int)nl) {
                        uint32_t *dst = (uint32_t *)(kWT ? wt.recv(r) : p.rk.recv[r]) + q * PW;
                        if constexpr (PW == 1)
                            __hip_atomic_store(dst, y[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            __hip_atomic_store((uint64_t *)dst, ((uint64_t)y[1] << 32) | y[0],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            } else {
                const bool word = PW == 2 && p.tail_bytes >= 4;
                for (int r = 0; r < (int)nl; ++r) {
                    uint32_t *dst = (uint32_t *)p.rk.recv[r] + q * PW;
                    if (word)
                        dst[0] = y[0];
                    if (p.tail_bytes & 2u)
                        ((uint16_t *)dst)[word ? 2 : 0] = (uint16_t)y[word ? PW - 1 : 0];
                }
            }
        }
    }
}

// Clears the async-error word and all packets, and sets every sequence-table
// entry to `seq0` (vector stores; no memset node in graphs).
__global__ __launch_bounds__(256) void ll_reset(uint64_t *pkts, uint64_t npkts, uint32_t *seq,
                                                uint64_t nseq, uint32_t seq0, uint32_t *ctrl)
{
    const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = i0; i < npkts; i += step)
        pkts[i] = 0;
    for (uint64_t i = i0; i < nseq; i += step)
        seq[i] = seq0;
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

template <typename T, int RMAX, bool EXACT, int PW, bool SEQ, int NODE>
hipError_t launch_table(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int want_threads, uint64_t want_blocks, int group,
                        hipStream_t stream)
{
    LLParams<RMAX> p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    const uint64_t bytes = (uint64_t)count * T::kBytes;
    p.npkt = (bytes + 4 * PW - 1) / (4 * PW);
    p.tail_bytes = (uint32_t)(bytes % (4 * PW));
    p.pkts = comm->pkts;
    p.pkt_stride = comm->pkt_stride / PW;
    p.region_bytes = (uint64_t)comm->max_ranks * comm->pkt_stride * sizeof(uint64_t);
    p.ctrl = comm->ctrl;
    p.seq = comm->seq;
    p.seq_stride = (uint64_t)comm->max_ranks;
    p.nranks = (uint32_t)nranks;
    p.node_starts = 0u;
    if constexpr (NODE == kNodeMask)
        for (int j = group; j < nranks; j += group)
            p.node_starts |= 1u << j;
    p.flag_skew = (uint32_t)comm->opt[arOptDebugFlagSkew];
    p.timeout_ticks = (uint64_t)comm->opt[arOptPollTimeoutUs] * comm->wall_clock_khz / 1000u;

    // Launch shape: the caller's, else the measured default for the rank
    // count and size.  With only the workgroup size given, the default's
    // lanes per rank are kept.
    const LLShape d = ll_default_shape(nranks, bytes);
    int threads = want_threads;
    if (threads <= 0)
        threads = d.threads;
    if (threads > ll_max_threads(RMAX))
        threads = ll_max_threads(RMAX);
    const int resident =
        comm->ll_resident[ll_kind(SEQ, NODE)][PW - 1][T::kId][EXACT ? variant_of(RMAX) : kRankVariants]
                         [thread_index(threads)];
    uint64_t max_per_rank = (uint64_t)(resident / nranks);
    if (max_per_rank < 1)
        max_per_rank = 1;

    uint64_t per_rank = want_blocks;
    if (per_rank == 0)
        per_rank = ((uint64_t)d.per_rank * (uint64_t)d.threads + (uint64_t)threads - 1) /
                   (uint64_t)threads;
    if (per_rank > max_per_rank)
        per_rank = max_per_rank;
    if (per_rank > p.npkt)
        per_rank = p.npkt;
    if (per_rank < 1)
        per_rank = 1;
    p.put_per_block = (p.npkt + per_rank - 1) / per_rank;
    p.get_per_block = (p.put_per_block + (uint64_t)nranks - 1) / (uint64_t)nranks;
    if constexpr (SEQ) {
        // Every sub-slice starts on a group boundary and spans whole groups,
        // so each group is consumed by one wave (threads is a multiple of 64).
        // That can only lower the workgroup count.
        const uint64_t G = seq_group(PW);
        p.get_per_block = (p.get_per_block + G - 1) / G * G;
        p.put_per_block = p.get_per_block * (uint64_t)nranks;
        per_rank = (p.npkt + p.put_per_block - 1) / p.put_per_block;
    }
    p.blocks_per_rank = (uint32_t)per_rank;
    const uint32_t grid = (uint32_t)(per_rank * (uint64_t)nranks);

    comm->last = {arProtoLL, 1, grid, (uint32_t)threads, 8 * PW, 0,
                  NODE == kNodeFlat ? 0 : group, 0, 4 * PW};
    hipLaunchKernelGGL((ll_oneshot<T, RMAX, EXACT, PW, SEQ, NODE>), dim3(grid), dim3(threads), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename T, int PW, bool SEQ, int G>
hipError_t launch_dtype(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int th, uint64_t bl, int grp, hipStream_t stream)
{
    switch (nranks) {
    case 1: return launch_table<T, 1, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 2: return launch_table<T, 2, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 4: return launch_table<T, 4, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 8: return launch_table<T, 8, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 16: return launch_table<T, 16, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 32: return launch_table<T, 32, true, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    default: break;
    }
    // Other rank counts: the next larger table, with the count at run time.
    if (nranks < 4)
        return launch_table<T, 4, false, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    if (nranks < 8)
        return launch_table<T, 8, false, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    if (nranks < 16)
        return launch_table<T, 16, false, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
    return launch_table<T, 32, false, PW, SEQ, G>(send, recv, count, nranks, comm, th, bl, grp, stream);
}

// The hierarchical order.  A power-of-two rank count has power-of-two node
// sizes only (a node size divides the rank count), each compiled in; any
// other rank count takes the bitmask kernel.
template <typename T, int PW, int RMAX, int NODE>
hipError_t launch_nodes(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int th, uint64_t bl, int grp, hipStream_t stream)
{
    if constexpr (NODE < RMAX) {
        if (grp == NODE)
            return launch_table<T, RMAX, true, PW, false, NODE>(send, recv, count, nranks, comm,
                                                                 th, bl, grp, stream);
        return launch_nodes<T, PW, RMAX, NODE * 2>(send, recv, count, nranks, comm, th, bl, grp,
                                                   stream);
    } else {
        return launch_table<T, 32, false, PW, false, kNodeMask>(send, recv, count, nranks, comm,
                                                                th, bl, grp, stream);
    }
}

template <typename T, int PW>
hipError_t launch_grouped(const void *const *send, void *const *recv, size_t count, int nranks,
                          const arComm *comm, int th, uint64_t bl, int grp, hipStream_t stream)
{
    switch (nranks) {
    case 4: return launch_nodes<T, PW, 4, 2>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 8: return launch_nodes<T, PW, 8, 2>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 16: return launch_nodes<T, PW, 16, 2>(send, recv, count, nranks, comm, th, bl, grp, stream);
    case 32: return launch_nodes<T, PW, 32, 2>(send, recv, count, nranks, comm, th, bl, grp, stream);
    default:
        return launch_table<T, 32, false, PW, false, kNodeMask>(send, recv, count, nranks, comm,
                                                                th, bl, grp, stream);
    }
}

template <typename T>
hipError_t launch_width(const void *const *send, void *const *recv, size_t count, int nranks,
                        const arComm *comm, int th, uint64_t bl, int pkt_bytes, int scheme,
                        int group, hipStream_t stream)
{
    const bool seq = scheme == kSchemeSequenced;
    constexpr int F = kNodeFlat;
    // The hierarchical order is compiled for the cleared scheme only (the
    // caller rejects it with the sequenced one).
    if (group != 0)
        return pkt_bytes == 16
                   ? launch_grouped<T, 2>(send, recv, count, nranks, comm, th, bl, group, stream)
                   : launch_grouped<T, 1>(send, recv, count, nranks, comm, th, bl, group, stream);
    if (pkt_bytes == 16)
        return seq ? launch_dtype<T, 2, true, F>(send, recv, count, nranks, comm, th, bl, 0, stream)
                   : launch_dtype<T, 2, false, F>(send, recv, count, nranks, comm, th, bl, 0, stream);
    return seq ? launch_dtype<T, 1, true, F>(send, recv, count, nranks, comm, th, bl, 0, stream)
               : launch_dtype<T, 1, false, F>(send, recv, count, nranks, comm, th, bl, 0, stream);
}

template <typename T, int RMAX, bool EXACT, int PW, bool SEQ, int G>
hipError_t query_one(int *out)
{
    for (int i = 0; i < kThreadChoices; ++i) {
        if (kThreadOptions[i] > ll_max_threads(RMAX)) {
            out[i] = 0;  // never launched with this many threads
            continue;
        }
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&ll_oneshot<T, RMAX, EXACT, PW, SEQ, G>),
            kThreadOptions[i], 0);
        if (e != hipSuccess)
            return e;
        out[i] = per_cu;
    }
    return hipSuccess;
}

template <typename T, int PW, bool SEQ, int G>
hipError_t query_dtype(int (*tab)[kThreadChoices])
{
    hipError_t e;
    if ((e = query_one<T, 1, true, PW, SEQ, G>(tab[0])) != hipSuccess) return e;
    if ((e = query_one<T, 2, true, PW, SEQ, G>(tab[1])) != hipSuccess) return e;
    if ((e = query_one<T, 4, true, PW, SEQ, G>(tab[2])) != hipSuccess) return e;
    if ((e = query_one<T, 8, true, PW, SEQ, G>(tab[3])) != hipSuccess) return e;
    if ((e = query_one<T, 16, true, PW, SEQ, G>(tab[4])) != hipSuccess) return e;
    if ((e = query_one<T, 32, true, PW, SEQ, G>(tab[5])) != hipSuccess) return e;
    // one entry for the four generic tables: the smallest of their counts
    int g[4][kThreadChoices] = {};
    if ((e = query_one<T, 4, false, PW, SEQ, G>(g[0])) != hipSuccess) return e;
    if ((e = query_one<T, 8, false, PW, SEQ, G>(g[1])) != hipSuccess) return e;
    if ((e = query_one<T, 16, false, PW, SEQ, G>(g[2])) != hipSuccess) return e;
    if ((e = query_one<T, 32, false, PW, SEQ, G>(g[3])) != hipSuccess) return e;
    for (int i = 0; i < kThreadChoices; ++i) {
        tab[6][i] = g[0][i];
        for (int t = 1; t < 4; ++t)
            tab[6][i] = g[t][i] < tab[6][i] ? g[t][i] : tab[6][i];
    }
    return hipSuccess;
}

template <int PW, bool SEQ, int G>
hipError_t query_width(int (*tab)[kRankVariants + 1][kThreadChoices])
{
    hipError_t e;
    if ((e = query_dtype<Bf16, PW, SEQ, G>(tab[kBf16])) != hipSuccess) return e;
    if ((e = query_dtype<Fp16, PW, SEQ, G>(tab[kFp16])) != hipSuccess) return e;
    return query_dtype<Fp32, PW, SEQ, G>(tab[kFp32]);
}

// The hierarchical-order kernels that launch_grouped can pick: nodes of NODE
// ranks at each power-of-two rank count above NODE, or the bitmask kernel.
template <typename T, int PW, int NODE>
hipError_t query_nodes(int (*tab)[kThreadChoices])
{
    if constexpr (NODE == kNodeMask) {
        return query_one<T, 32, false, PW, false, kNodeMask>(tab[kRankVariants]);
    } else {
        hipError_t e;
        if constexpr (NODE < 4)
            if ((e = query_one<T, 4, true, PW, false, NODE>(tab[2])) != hipSuccess) return e;
        if constexpr (NODE < 8)
            if ((e = query_one<T, 8, true, PW, false, NODE>(tab[3])) != hipSuccess) return e;
        if constexpr (NODE < 16)
            if ((e = query_one<T, 16, true, PW, false, NODE>(tab[4])) != hipSuccess) return e;
        return query_one<T, 32, true, PW, false, NODE>(tab[5]);
    }
}

template <int NODE>
hipError_t query_grouped(int (*tab)[3][kRankVariants + 1][kThreadChoices])
{
    hipError_t e;
    if ((e = query_nodes<Bf16, 1, NODE>(tab[0][kBf16])) != hipSuccess) return e;
    if ((e = query_nodes<Fp16, 1, NODE>(tab[0][kFp16])) != hipSuccess) return e;
    if ((e = query_nodes<Fp32, 1, NODE>(tab[0][kFp32])) != hipSuccess) return e;
    if ((e = query_nodes<Bf16, 2, NODE>(tab[1][kBf16])) != hipSuccess) return e;
    if ((e = query_nodes<Fp16, 2, NODE>(tab[1][kFp16])) != hipSuccess) return e;
    return query_nodes<Fp32, 2, NODE>(tab[1][kFp32]);
}

}  // namespace

hipError_t launch_ll(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const arComm *comm, int threads, uint64_t blocks, int pkt_bytes,
                     int scheme, int group, hipStream_t stream)
{
    switch (dtype) {
    case kBf16:
        return launch_width<Bf16>(send, recv, count, nranks, comm, threads, blocks, pkt_bytes,
                                  scheme, group, stream);
    case kFp16:
        return launch_width<Fp16>(send, recv, count, nranks, comm, threads, blocks, pkt_bytes,
                                  scheme, group, stream);
    default:
        return launch_width<Fp32>(send, recv, count, nranks, comm, threads, blocks, pkt_bytes,
                                  scheme, group, stream);
    }
}

hipError_t launch_reset(const arComm *comm, hipStream_t stream)
{
    const uint64_t npkts = (uint64_t)comm->max_ranks * comm->pkt_stride;
    const uint64_t most = npkts > comm->seq_words ? npkts : comm->seq_words;
    uint64_t blocks = (most + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(ll_reset, dim3((uint32_t)blocks), dim3(256), 0, stream, comm->pkts, npkts,
                       comm->seq, comm->seq_words, (uint32_t)comm->opt[arOptDebugSeqStart],
                       comm->ctrl);
    return hipGetLastError();
}

hipError_t query_ll_residency(arComm *comm)
{
    int per_cu[kLLKinds][2][3][kRankVariants + 1][kThreadChoices] = {};
    hipError_t e;
    constexpr int F = kNodeFlat;
    if ((e = query_width<1, false, F>(per_cu[ll_kind(false, F)][0])) != hipSuccess) return e;
    if ((e = query_width<2, false, F>(per_cu[ll_kind(false, F)][1])) != hipSuccess) return e;
    if ((e = query_width<1, true, F>(per_cu[ll_kind(true, F)][0])) != hipSuccess) return e;
    if ((e = query_width<2, true, F>(per_cu[ll_kind(true, F)][1])) != hipSuccess) return e;
    if ((e = query_grouped<kNodeMask>(per_cu[ll_kind(false, kNodeMask)])) != hipSuccess) return e;
    if ((e = query_grouped<2>(per_cu[ll_kind(false, 2)])) != hipSuccess) return e;
    if ((e = query_grouped<4>(per_cu[ll_kind(false, 4)])) != hipSuccess) return e;
    if ((e = query_grouped<8>(per_cu[ll_kind(false, 8)])) != hipSuccess) return e;
    if ((e = query_grouped<16>(per_cu[ll_kind(false, 16)])) != hipSuccess) return e;
    if ((e = query_ll_dense_residency(per_cu[kLLDenseKind][0])) != hipSuccess) return e;
    for (int s = 0; s < kLLKinds; ++s)
        for (int w = 0; w < 2; ++w)
            for (int d = 0; d < 3; ++d)
                for (int v = 0; v <= kRankVariants; ++v)
                    for (int t = 0; t < kThreadChoices; ++t)
                        comm->ll_resident[s][w][d][v][t] = per_cu[s][w][d][v][t] * comm->cu_count;
    return hipSuccess;
}

}  // namespace ar
