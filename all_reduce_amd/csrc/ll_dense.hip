// ll_dense.hip -- the LL one-shot with three-element packets for 16-bit types.
//
// The LL protocol of "MSCCL++：让 GPU 通信像 CUDA 一样可编程"
// (infinitensor.com/news/50, "MemoryChannel") pays for its fine-grained
// synchronisation in bandwidth: every payload byte also moves a flag.  With
// the word packet of ll_oneshot.hip ({4-byte payload, 4-byte flag}, one
// 64-bit atomic store), half of every packet is flag, and a call writes
// packets, then zeroes them, then writes the outputs: 2.5 times the bytes of
// the outputs alone.  On MI355X that write traffic is what bounds LL from a
// few hundred KiB per rank up (rocprofv3 counts exactly packets + clears +
// outputs in the L2-to-fabric writes).
//
// For bfloat16 and float16 this kernel packs three elements and a 16-bit flag
// into the same 8-byte packet: bits 0-47 hold elements 3p, 3p+1, 3p+2 of the
// rank's buffer, bits 48-63 the flag.  It is still one 64-bit atomic store,
// so a reader that sees the flag sees the three elements; 75 % of the packet
// is payload, a third fewer packet and clear bytes than the word packet.
//
// Elements sit at a 6-byte stride in the packets but a 2-byte stride in the
// buffers, so each wave stages its data through a private piece of LDS:
//   put     a wave loads 512 packets' worth of its rank's elements (3 KiB)
//           with coalesced 16-byte loads, writes them to LDS, and reads back
//           three elements per packet, so that its packet stores are
//           coalesced too (64 consecutive packets per store instruction);
//   poll    as in ll_oneshot.hip: per lane, R packets per packet index,
//           re-read until every flag is ready (wall-clock and re-read
//           bounds), then reduced in binary32 in rank order 0..R-1 from
//           rank 0's value and rounded once, and the R packets cleared;
//   output  the wave's three-element results go to LDS and out again as
//           8-byte words at consecutive addresses per lane, stored to all R
//           receive buffers at agent scope.
// Every LDS exchange stays inside one wave (no workgroup barrier inside
// loops whose trip counts differ between waves); the loops are wave-uniform
// and each exchange is fenced at wavefront scope.
//
// Slices and sub-slices are whole multiples of 8 packets (24 elements, 48
// bytes), so every wave's output range starts on a 16-byte boundary.  Flags:
// the cleared scheme of ll_oneshot.hip (packet memory is zero between calls;
// a packet is ready when its flag is 0xffff; the reader zeroes what it
// read), so calls of either packet format may follow each other.  The same
// co-residency requirement holds: the host caps the grid with the occupancy
// calculator, which counts this kernel's LDS.
#include "ar_internal.hpp"
#include "ll_packet.hpp"

namespace ar {

template <int R>
struct LLDenseParams {
    RankTable<R> rk;
    uint64_t *pkts;          // packet scratch; rank k's packets start at k * pkt_stride
    uint64_t pkt_stride;     // 8-byte packets per rank region
    uint64_t count;          // elements per rank
    uint64_t npkt;           // packets per rank = ceil(count / 3)
    uint64_t put_per_block;  // packets each workgroup publishes for its rank (a multiple of 8)
    uint64_t get_per_block;  // packets each workgroup polls (a multiple of 8)
    uint32_t *ctrl;          // [0] async error (0 or arTimeout)
    uint64_t timeout_ticks;  // wall-clock ticks one packet wait may take
    uint32_t flag_skew;      // test hook: consumers wait for flag + skew
    uint32_t nranks;
};

constexpr int kDensePutPackets = 512;                 // per wave and round: 8 per lane
constexpr int kDensePutVecs = kDensePutPackets * 6 / 16;  // 192 16-byte vectors: 3 per lane
constexpr uint32_t kDenseReady = 0xffffu;
constexpr int kDenseMaxThreads = 512;
// Packet indices a lane polls at once (R packets each), as in ll_oneshot.hip.
constexpr int dense_get_batch(int rmax) { return rmax <= 8 ? 2 : 1; }
// LDS per wave: the put staging (3 KiB) is the larger of the two uses.
constexpr int kDenseStageWords = kDensePutVecs * 4;
constexpr size_t dense_lds_bytes(int threads) { return (size_t)(threads / 64) * kDenseStageWords * 4; }

// Wave-scope ordering of this lane's LDS accesses against the other lanes':
// the hardware runs a wave's LDS instructions in order, and the fences keep
// the compiler from moving LDS loads or stores across the exchange point.
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 48 payload bits of packet `rel` of a put round: its three elements sit
// at bytes [6 rel, 6 rel + 6) of the staged data, read as the two aligned
// 32-bit words that cover them (no unaligned LDS access).
__device__ inline uint64_t staged_payload(const uint32_t *stage, uint32_t rel)
{
    const uint32_t wi = (rel * 6) >> 2;
    const uint32_t w0 = stage[wi], w1 = stage[wi + 1];
    return (rel & 1u) ? (uint64_t)__builtin_amdgcn_alignbit(w1, w0, 16) | ((uint64_t)(w1 >> 16) << 32)
                      : (uint64_t)w0 | ((uint64_t)(w1 & 0xffffu) << 32);
}

template <typename T, int RMAX, bool EXACT>
__global__ __launch_bounds__(kDenseMaxThreads) void ll_dense(LLDenseParams<RMAX> p)
{
    static_assert(T::kBytes == 2, "three-element packets hold 16-bit elements");
    constexpr int GB = dense_get_batch(RMAX);
    extern __shared__ uint32_t dense_stage[];  // kDenseStageWords per wave
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t nwaves = blockDim.x >> 6;
    uint32_t *stage = dense_stage + wave * kDenseStageWords;
    const uint32_t k = blockIdx.x % n;
    const uint32_t b = blockIdx.x / n;
    const uint64_t bytes = p.count * 2;
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

    // ---- put: rank k's packets [p0, p1) of slice b ----------------------
    const uint64_t p0 = (uint64_t)b * p.put_per_block;
    const uint64_t p1 = (p0 + p.put_per_block < p.npkt) ? p0 + p.put_per_block : p.npkt;
    const uint8_t *src = (const uint8_t *)p.rk.send[k];
    uint64_t *mine = p.pkts + (uint64_t)k * p.pkt_stride;
    for (uint64_t base = p0 + (uint64_t)wave * kDensePutPackets; base < p1;
         base += (uint64_t)nwaves * kDensePutPackets) {
        // the round's elements [3 base, 3 base + 1536): bytes [6 base, +3072),
        // 16-byte aligned because base is a multiple of 8
        const uint64_t byte0 = base * 6;
        u32x4 v[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const uint64_t at = byte0 + (uint64_t)(lane + 64 * j) * 16;
            if (at + 16 <= bytes) {
                v[j] = *(const u32x4 *)(src + at);
            } else {
                // the message's last, partial vector (or past its end): the
                // elements that exist, zeros for the rest
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (uint32_t e = 0; e < 8 && at + 2 * e < bytes; ++e)
                    w[e >> 1] |= (uint32_t)((const uint16_t *)(src + at))[e] << (16 * (e & 1));
                v[j] = {w[0], w[1], w[2], w[3]};
            }
        }
        wave_lds_sync();  // the previous round's LDS reads are done
#pragma unroll
        for (int j = 0; j < 3; ++j)
            *(u32x4 *)(stage + (lane + 64 * j) * 4) = v[j];
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t rel = lane + 64u * j;  // packet within the round
            const uint64_t q = base + rel;
            if (q < p1) {
                const uint64_t pkt = staged_payload(stage, rel) | ((uint64_t)kDenseReady << 48);
                __hip_atomic_store(mine + q, pkt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // ---- poll, reduce, clear, output: sub-slice k of slice b --------------
    const uint32_t want = kDenseReady - p.flag_skew;
    const uint64_t g0 = p0 + (uint64_t)k * p.get_per_block;
    const uint64_t g1 = (g0 + p.get_per_block < p1) ? g0 + p.get_per_block : p1;
    // valid output elements of this sub-slice end at min(3 g1, count)
    const uint64_t elem_end = (3 * g1 < p.count) ? 3 * g1 : p.count;
    uint64_t wait_start = 0;
    uint64_t spins = 0;
    bool gave_up = false;
    constexpr uint32_t kRound = 64u * GB;  // packet indices per wave and round
    for (uint64_t qb = g0 + (uint64_t)wave * kRound; qb < g1; qb += (uint64_t)nwaves * kRound) {
        // (the run-time rank count re-read each round, as in ll_oneshot.hip)
        uint32_t nl = n;
        if constexpr (kWT) {
            wt.refresh();
            if constexpr (!EXACT)
                asm volatile("" : "+s"(nl));
        }
        uint64_t pk[GB][RMAX];
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = qb + lane + 64u * v;
            if (q < g1 && !gave_up)
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    if (EXACT || j < (int)nl)
                        pk[v][j] = read_packet(p.pkts + (uint64_t)j * p.pkt_stride + q);
        }
        if (!gave_up) {
            for (;;) {
                bool ready = true;
#pragma unroll
                for (int v = 0; v < GB; ++v)
                    if (qb + lane + 64u * v < g1)
#pragma unroll
                        for (int j = 0; j < RMAX; ++j)
                            if (EXACT || j < (int)nl)
                                ready = ready && (uint32_t)(pk[v][j] >> 48) == want;
                if (ready)
                    break;
                const uint64_t now = wall_clock64();
                if (wait_start == 0)
                    wait_start = now;
                else if (now - wait_start > p.timeout_ticks || ++spins > p.timeout_ticks) {
                    __hip_atomic_store(p.ctrl + 0, (uint32_t)arTimeout, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    gave_up = true;
                    break;
                }
#pragma unroll
                for (int v = 0; v < GB; ++v) {
                    const uint64_t q = qb + lane + 64u * v;
                    if (q < g1)
#pragma unroll
                        for (int j = 0; j < RMAX; ++j)
                            if ((EXACT || j < (int)nl) && (uint32_t)(pk[v][j] >> 48) != want)
                                pk[v][j] = read_packet(p.pkts + (uint64_t)j * p.pkt_stride + q);
                }
            }
        }
        // reduce in rank order, then clear what was read, then stage the
        // results.  Every index's sum is taken before the first clear: gfx9
        // counts loads and stores on one counter, so a packet value used after
        // a store would make the wave wait for that store's completion too.
        uint32_t y01[GB], y2[GB];
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = qb + lane + 64u * v;
            y01[v] = 0u;
            y2[v] = 0u;
            if (q < g1 && !gave_up) {
                float a[4];
                T::widen((uint32_t)pk[v][0], a);
                T::widen((uint32_t)(pk[v][0] >> 32) & 0xffffu, a + 2);
#pragma unroll
                for (int j = 1; j < RMAX; ++j) {
                    if (EXACT || j < (int)nl) {
                        float x[4];
                        T::widen((uint32_t)pk[v][j], x);
                        T::widen((uint32_t)(pk[v][j] >> 32) & 0xffffu, x + 2);
                        a[0] = a[0] + x[0];
                        a[1] = a[1] + x[1];
                        a[2] = a[2] + x[2];
                    }
                }
                a[3] = 0.0f;
                y01[v] = T::narrow(a);
                y2[v] = T::narrow(a + 2) & 0xffffu;
            }
        }
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint64_t q = qb + lane + 64u * v;
            if (q < g1 && !gave_up)
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    if (EXACT || j < (int)nl)
                        put_packet(p.pkts + (uint64_t)j * p.pkt_stride + q, 0u, 0u);
        }
        wave_lds_sync();  // the previous round's output reads are done
        // index rel's three results go to bytes [6 rel, 6 rel + 6), in
        // naturally aligned pieces: a word then a half for even rel, a half
        // then a word for odd rel
        uint16_t *s16 = (uint16_t *)stage;
#pragma unroll
        for (int v = 0; v < GB; ++v) {
            const uint32_t rel = lane + 64u * v;
            if ((rel & 1u) == 0) {
                stage[rel * 6 / 4] = y01[v];
                s16[rel * 3 + 2] = (uint16_t)y2[v];
            } else {
                s16[rel * 3] = (uint16_t)y01[v];
                stage[(rel * 6 + 2) / 4] = (y01[v] >> 16) | (y2[v] << 16);
            }
        }
        wave_lds_sync();
        // the round's results leave as 8-byte words, word i holding elements
        // [3 qb + 4 i, +4): consecutive lanes store consecutive words, so each
        // store instruction writes whole lines of every receive buffer
        const uint64_t e0 = 3 * qb;
        for (uint32_t i = lane; i < 48u * GB; i += 64u) {
            const uint64_t e = e0 + 4u * i;
            if (e >= elem_end)
                continue;
            if (e + 4 <= elem_end) {
                const uint64_t y = ((const uint64_t *)stage)[i];
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (EXACT || r < (int)nl)
                        __hip_atomic_store((uint64_t *)((uint8_t *)(kWT ? wt.recv(r) : p.rk.recv[r]) + e * 2), y,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                // the message's last, partial word: its elements one by one
                const uint16_t *ys = (const uint16_t *)stage + 4 * i;
                for (int r = 0; r < (int)nl; ++r)
                    for (uint64_t t = e; t < elem_end; ++t)
                        ((uint16_t *)p.rk.recv[r])[t] = ys[t - e];
            }
        }
    }
}

namespace {

constexpr int kDenseThreadOptions[kThreadChoices] = {64, 128, 256, 512, 1024};

int dense_thread_index(int threads)
{
    for (int i = 0; i < kThreadChoices; ++i)
        if (kDenseThreadOptions[i] == threads)
            return i;
    return 2;
}

int dense_variant(int nranks)
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
    LLDenseParams<RMAX> p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    p.count = count;
    p.npkt = (count + 2) / 3;
    p.pkts = comm->pkts;
    p.pkt_stride = comm->pkt_stride;
    p.ctrl = comm->ctrl;
    p.nranks = (uint32_t)nranks;
    p.flag_skew = (uint32_t)comm->opt[arOptDebugFlagSkew];
    p.timeout_ticks = (uint64_t)comm->opt[arOptPollTimeoutUs] * comm->wall_clock_khz / 1000u;

    const LLShape d = ll_dense_default_shape(nranks, (uint64_t)count * 2);
    int threads = want_threads > 0 ? want_threads : d.threads;
    if (threads > kDenseMaxThreads)
        threads = kDenseMaxThreads;
    const int resident = comm->ll_resident[kLLDenseKind][0][T::kId][EXACT ? dense_variant(RMAX)
                                                                          : kRankVariants]
                                          [dense_thread_index(threads)];
    uint64_t max_per_rank = (uint64_t)(resident / nranks);
    if (max_per_rank < 1)
        max_per_rank = 1;
    uint64_t per_rank = want_blocks;
    if (per_rank == 0)
        per_rank = ((uint64_t)d.per_rank * (uint64_t)d.threads + (uint64_t)threads - 1) /
                   (uint64_t)threads;
    if (per_rank > max_per_rank)
        per_rank = max_per_rank;
    if (per_rank < 1)
        per_rank = 1;
    // Whole groups of 8 packets per sub-slice (16-byte aligned output
    // ranges); that can only lower the workgroup count.
    uint64_t put = (p.npkt + per_rank - 1) / per_rank;
    uint64_t get = (put + (uint64_t)nranks - 1) / (uint64_t)nranks;
    get = (get + 7) / 8 * 8;
    p.get_per_block = get;
    p.put_per_block = get * (uint64_t)nranks;
    per_rank = (p.npkt + p.put_per_block - 1) / p.put_per_block;
    const uint32_t grid = (uint32_t)(per_rank * (uint64_t)nranks);

    comm->last = {arProtoLL, 1, grid, (uint32_t)threads, 8, 0, 0, 0, 6};
    hipLaunchKernelGGL((ll_dense<T, RMAX, EXACT>), dim3(grid), dim3(threads),
                       dense_lds_bytes(threads), stream, p);
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
    default: break;
    }
    // Other rank counts: the next larger table, with the count at run time.
    if (nranks < 4)
        return launch_table<T, 4, false>(send, recv, count, nranks, comm, th, bl, stream);
    if (nranks < 8)
        return launch_table<T, 8, false>(send, recv, count, nranks, comm, th, bl, stream);
    if (nranks < 16)
        return launch_table<T, 16, false>(send, recv, count, nranks, comm, th, bl, stream);
    return launch_table<T, 32, false>(send, recv, count, nranks, comm, th, bl, stream);
}

template <typename T, int RMAX, bool EXACT>
hipError_t query_one(int *out)
{
    for (int i = 0; i < kThreadChoices; ++i) {
        if (kDenseThreadOptions[i] > kDenseMaxThreads) {
            out[i] = 0;
            continue;
        }
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&ll_dense<T, RMAX, EXACT>),
            kDenseThreadOptions[i], dense_lds_bytes(kDenseThreadOptions[i]));
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
    // one entry for the four generic tables: the smallest of their counts
    int g[4][kThreadChoices] = {};
    if ((e = query_one<T, 4, false>(g[0])) != hipSuccess) return e;
    if ((e = query_one<T, 8, false>(g[1])) != hipSuccess) return e;
    if ((e = query_one<T, 16, false>(g[2])) != hipSuccess) return e;
    if ((e = query_one<T, 32, false>(g[3])) != hipSuccess) return e;
    for (int i = 0; i < kThreadChoices; ++i) {
        tab[6][i] = g[0][i];
        for (int t = 1; t < 4; ++t)
            tab[6][i] = g[t][i] < tab[6][i] ? g[t][i] : tab[6][i];
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_ll_dense(const void *const *send, void *const *recv, size_t count, int dtype,
                           int nranks, const arComm *comm, int threads, uint64_t blocks,
                           hipStream_t stream)
{
    return dtype == kBf16
               ? launch_dtype<Bf16>(send, recv, count, nranks, comm, threads, blocks, stream)
               : launch_dtype<Fp16>(send, recv, count, nranks, comm, threads, blocks, stream);
}

hipError_t query_ll_dense_residency(int (*per_cu)[kRankVariants + 1][kThreadChoices])
{
    hipError_t e;
    if ((e = query_dtype<Bf16>(per_cu[kBf16])) != hipSuccess)
        return e;
    return query_dtype<Fp16>(per_cu[kFp16]);
}

}  // namespace ar
