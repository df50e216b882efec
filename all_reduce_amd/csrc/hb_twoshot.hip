// hb_twoshot.hip -- the high-bandwidth (HB) all-reduce: two-shot, by chunk.
//
// The HB protocol of the MemoryChannel table in "MSCCL++：让 GPU 通信像 CUDA
// 一样可编程" (infinitensor.com/news/50) moves large blocks with few
// synchronisations, for prefill-size messages; SGLang's native
// default_allreduce_rsag_zero_copy ("SGLang 中的 MSCCL++ All-Reduce 基准测试与
// 推理集成指南", blog.gitcode.com, section 4.4) names its shape: a
// reduce-scatter followed by an all-gather, straight between user buffers.
//
// On one GPU the R ranks' buffers are all local, so both shots fuse per tile:
//   reduce-scatter  the workgroups of simulated rank c own chunk c
//                   (vectors [c*C, (c+1)*C), the last chunk takes the rest) and
//                   read that chunk from all R send buffers with 128-bit loads;
//   reduce          binary32 accumulation in registers, rank order 0..R-1;
//   all-gather      the reduced vector goes straight from registers to all R
//                   receive buffers with 128-bit stores.
// No flag and no barrier is needed: a lane loads all R inputs of a position
// before it stores any output of that position, and positions are disjoint
// between lanes, so in-place (recv[r] == send[r]) is safe too.
//
// The work is HBM-streaming: 2 * R * bytes-per-rank per call, about 0.22 flop
// per byte at R = 8 in bf16, far below the ridge point; no LDS, no MFMA.
// Workgroup w serves chunk w % R, so consecutive workgroups -- which the
// dispatcher spreads round-robin over the 8 XCDs -- stream different chunks.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

// Two-shot HB launch parameters.
template <int R>
struct HBParams {
    RankTable<R> rk;
    uint64_t nvec;        // whole 16-byte vectors per rank
    uint64_t chunk_vec;   // vectors per chunk 0..R-2; the last chunk takes the rest
    uint32_t blocks_per_chunk;
    uint32_t nranks;      // runtime rank count (the generic kernel; else == R)
    uint32_t tail_elems;  // elements after the last whole vector
    uint32_t interleaved; // 0: chunk c = contiguous vectors; 1: tiles c, c+R, c+2R, ...
    uint32_t group;       // hierarchical order: ranks per node (1 < group < nranks); else 0
    uint32_t pad;
};

// Scalar path for the elements after the last whole 16-byte vector.
template <typename T>
__device__ inline float load_elem(const void *base, uint64_t i)
{
    uint32_t w = (T::kBytes == 2) ? (uint32_t)((const uint16_t *)base)[i]
                                  : ((const uint32_t *)base)[i];
    float f[T::kPerWord];
    T::widen(w, f);
    return f[0];
}

template <typename T>
__device__ inline void store_elem(void *base, uint64_t i, float a)
{
    float f[T::kPerWord] = {};
    f[0] = a;
    uint32_t w = T::narrow(f);
    if constexpr (T::kBytes == 2)
        ((uint16_t *)base)[i] = (uint16_t)w;
    else
        ((uint32_t *)base)[i] = w;
}

// A vector of -0 in the element type, loaded by a generic table's slots past
// the rank count: adding -0 leaves every binary32 value as it is.
__device__ u32x4 kNegZero16 = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
__device__ u32x4 kNegZero32 = {0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u};
template <typename T>
__device__ inline const u32x4 *neg_zero_vec()
{
    return T::kBytes == 2 ? &kNegZero16 : &kNegZero32;
}

// Largest workgroup compiled for a rank-table size: the R 16-byte vectors a
// lane holds (4 VGPRs each) must fit the register share of that many threads.
constexpr int hb_max_threads(int rmax) { return rmax >= 32 ? 256 : (rmax >= 16 ? 512 : 1024); }

// RMAX: size of the rank table.  EXACT: nranks == RMAX at compile time;
// otherwise nranks < RMAX arrives at run time and ranks >= nranks are skipped.
// U: 16-byte vectors per lane per rank in flight.  NT: non-temporal access.
// NODE: summation order.  0 is the flat order 0..R-1.  Otherwise the
// hierarchical order: the ranks form nodes of consecutive ranks, each node's
// partial is summed in binary32 in rank order, then the partials in node
// order, then one rounding (what an all-reduce that reduces inside each node
// first and across nodes second computes, with binary32 cross-node partials).
// NODE > 0 fixes the node size at compile time, so that every fold below is
// placed by the compiler; NODE < 0 takes it from p.group at run time.
// The workgroup size is a launch parameter (a tile is blockDim.x * U vectors).
template <typename T, int RMAX, bool EXACT, int U, bool NT, int NODE>
__global__ __launch_bounds__(hb_max_threads(RMAX)) void hb_twoshot(HBParams<RMAX> p)
{
    constexpr bool kGrouped = NODE != 0;
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint32_t node = NODE > 0 ? (uint32_t)NODE : p.group;
    const uint32_t nthr = blockDim.x;
    const uint32_t c = blockIdx.x % n;       // chunk, and the simulated rank owning it
    const uint32_t bb = blockIdx.x / n;      // this workgroup's place among the chunk's
    const uint64_t tile = (uint64_t)nthr * U;
    // Chunk c is either the contiguous vectors [c*C, (c+1)*C) (the last chunk
    // takes the rest) or, interleaved, every tile whose index is c modulo n.
    uint64_t start, step, end;
    if (p.interleaved) {
        start = ((uint64_t)bb * n + c) * tile;
        step = (uint64_t)p.blocks_per_chunk * n * tile;
        end = p.nvec;
    } else {
        const uint64_t c0 = (uint64_t)c * p.chunk_vec;
        start = c0 + (uint64_t)bb * tile;
        step = (uint64_t)p.blocks_per_chunk * tile;
        end = (c == n - 1) ? p.nvec : c0 + p.chunk_vec;
    }

    for (uint64_t base = start; base < end; base += step) {
        u32x4 v[U][RMAX];
        // reduce-scatter: every load of the tile is issued before any use
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * nthr + threadIdx.x;
            if (i < end) {
#pragma unroll
                for (int j = 0; j < RMAX; ++j) {
                    if constexpr (EXACT) {
                        v[u][j] = load16<NT>((const u32x4 *)p.rk.send[j] + i);
                    } else {
                        // Generic rank table: every slot loads, so that the
                        // loads issue back to back with no branch (and no
                        // wait) between them.  In the flat order a slot past
                        // the group loads a vector of -0 and is added like the
                        // others: x + (-0) is x for every binary32 x (signed
                        // zeros, subnormals, infinities; a NaN is already
                        // quiet after the group's own additions), and the
                        // sums need no per-rank branch (on MI355X 8-25 %
                        // faster at 2 KiB-1 MiB per rank, 3 to 24 ranks).  In
                        // the hierarchical order it rereads this lane's own
                        // vector of rank 0 -- an address the lane reads
                        // anyway and writes only after all its loads -- and
                        // is never accumulated.
                        const bool live = j < (int)n;
                        if constexpr (NODE == 0) {
                            const u32x4 *at = live ? (const u32x4 *)p.rk.send[j] + i
                                                   : neg_zero_vec<T>();
                            v[u][j] = load16<NT>(at);
                        } else {
                            const u32x4 *row = live ? (const u32x4 *)p.rk.send[j]
                                                    : (const u32x4 *)p.rk.send[0];
                            v[u][j] = load16<NT>(row + i);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * nthr + threadIdx.x;
            if (i < end) {
                u32x4 y;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float acc[T::kPerWord];
                    float total[T::kPerWord] = {};
                    T::widen(v[u][0][q], acc);
#pragma unroll
                    for (int j = 1; j < RMAX; ++j) {
                        if (EXACT || NODE == 0 || j < (int)n) {
                            float x[T::kPerWord];
                            T::widen(v[u][j][q], x);
                            if (kGrouped && (uint32_t)j % node == 0) {
                                // a node is complete: fold its partial in
#pragma unroll
                                for (int e = 0; e < T::kPerWord; ++e) {
                                    total[e] = (uint32_t)j == node ? acc[e] : total[e] + acc[e];
                                    acc[e] = x[e];
                                }
                            } else {
#pragma unroll
                                for (int e = 0; e < T::kPerWord; ++e)
                                    acc[e] = acc[e] + x[e];
                            }
                        }
                    }
                    if (kGrouped) {
#pragma unroll
                        for (int e = 0; e < T::kPerWord; ++e)
                            acc[e] = total[e] + acc[e];
                    }
                    y[q] = T::narrow(acc);
                }
                // all-gather: the reduced vector to every rank
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (EXACT || r < (int)n)
                        store16<NT>((u32x4 *)p.rk.recv[r] + i, y);
            }
        }
    }

    if (p.tail_elems != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < p.tail_elems) {
        constexpr uint64_t kPerVec = 16 / T::kBytes;
        const uint64_t i = p.nvec * kPerVec + threadIdx.x;
        float a = load_elem<T>(p.rk.send[0], i);
        float total = 0.0f;
        for (uint32_t j = 1; j < n; ++j) {
            const float x = load_elem<T>(p.rk.send[j], i);
            if (kGrouped && j % node == 0) {
                total = j == node ? a : total + a;
                a = x;
            } else {
                a = a + x;
            }
        }
        if (kGrouped)
            a = total + a;
        for (uint32_t r = 0; r < n; ++r)
            store_elem<T>(p.rk.recv[r], i, a);
    }
}

// The kernel above for a 32-rank table at one vector per lane, reading the
// table from a wave-held copy (WaveTable) instead of scalar registers, where
// 64 pointers do not fit: the compiler spills them and reloads them in blocks.
// Same chunks, same order of additions, same results.  On MI355X, bf16 and
// fp16: 3.6 against 4.8 us at 2 KiB per rank, 6.1 against 7.1 us at 512 KiB,
// 188-189 against 192-194 us at 16 MiB (24 ranks on the generic table, with
// its -0 slots: 4.1 against 6.4 us at 2 KiB); at 112 MiB per rank of fp32
// the scalar table is 1-2 % faster, so the launch
// takes this kernel up to kWaveTableMaxBytes per rank.  A separate kernel
// rather than a switch in the one above, whose code stays as it is.
template <typename T, bool EXACT, bool NT, int NODE>
__global__ __launch_bounds__(hb_max_threads(32)) void hb_twoshot_wave(HBParams<32> p)
{
    constexpr int RMAX = 32;
    constexpr bool kGrouped = NODE != 0;
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint32_t node = NODE > 0 ? (uint32_t)NODE : p.group;
    const uint32_t nthr = blockDim.x;
    const uint32_t c = blockIdx.x % n;
    const uint32_t bb = blockIdx.x / n;
    uint64_t start, step, end;
    if (p.interleaved) {
        start = ((uint64_t)bb * n + c) * nthr;
        step = (uint64_t)p.blocks_per_chunk * n * nthr;
        end = p.nvec;
    } else {
        const uint64_t c0 = (uint64_t)c * p.chunk_vec;
        start = c0 + (uint64_t)bb * nthr;
        step = (uint64_t)p.blocks_per_chunk * nthr;
        end = (c == n - 1) ? p.nvec : c0 + p.chunk_vec;
    }

    constexpr int U = 1;
    WaveTable<RMAX> wt(p.rk);
    for (uint64_t base = start; base < end; base += step) {
        // The table, the run-time rank count and the node size are re-read
        // each tile: hoisted out of the loop, the lane reads and the per-rank
        // tests would hold scalar registers across it again.
        wt.refresh();
        uint32_t nl = n, ndl = node;
        if constexpr (!EXACT)
            asm volatile("" : "+s"(nl));
        if constexpr (NODE < 0)
            asm volatile("" : "+s"(ndl));
        // The loop has hb_twoshot's shape, vector loop included: written more
        // compactly, the compiler interleaved the sums with the loads and
        // fewer loads were in flight (5 % slower at 16 MiB per rank).
        u32x4 v[U][RMAX];
        // reduce-scatter: every load of the tile is issued before any use
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * nthr + threadIdx.x;
            if (i < end) {
#pragma unroll
                for (int j = 0; j < RMAX; ++j)
                    // (slots past a generic table's count: as in hb_twoshot)
                    if constexpr (!EXACT && NODE == 0)
                        v[u][j] = load16<NT>(j < (int)nl ? (const u32x4 *)wt.send(j) + i
                                                          : neg_zero_vec<T>());
                    else
                        v[u][j] = load16<NT>((const u32x4 *)wt.send(EXACT || j < (int)nl ? j : 0) + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t i = base + (uint64_t)u * nthr + threadIdx.x;
            if (i < end) {
                u32x4 y;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float acc[T::kPerWord];
                    float total[T::kPerWord] = {};
                    T::widen(v[u][0][q], acc);
#pragma unroll
                    for (int j = 1; j < RMAX; ++j) {
                        if (EXACT || NODE == 0 || j < (int)nl) {
                            float x[T::kPerWord];
                            T::widen(v[u][j][q], x);
                            if (kGrouped && (uint32_t)j % ndl == 0) {
#pragma unroll
                                for (int e = 0; e < T::kPerWord; ++e) {
                                    total[e] = (uint32_t)j == ndl ? acc[e] : total[e] + acc[e];
                                    acc[e] = x[e];
                                }
                            } else {
#pragma unroll
                                for (int e = 0; e < T::kPerWord; ++e)
                                    acc[e] = acc[e] + x[e];
                            }
                        }
                    }
                    if (kGrouped) {
#pragma unroll
                        for (int e = 0; e < T::kPerWord; ++e)
                            acc[e] = total[e] + acc[e];
                    }
                    y[q] = T::narrow(acc);
                }
                // all-gather
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (EXACT || r < (int)nl)
                        store16<NT>((u32x4 *)wt.recv(r) + i, y);
            }
        }
    }

    if (p.tail_elems != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < p.tail_elems) {
        constexpr uint64_t kPerVec = 16 / T::kBytes;
        const uint64_t i = p.nvec * kPerVec + threadIdx.x;
        float a = load_elem<T>(p.rk.send[0], i);
        float total = 0.0f;
        for (uint32_t j = 1; j < n; ++j) {
            const float x = load_elem<T>(p.rk.send[j], i);
            if (kGrouped && j % node == 0) {
                total = j == node ? a : total + a;
                a = x;
            } else {
                a = a + x;
            }
        }
        if (kGrouped)
            a = total + a;
        for (uint32_t r = 0; r < n; ++r)
            store_elem<T>(p.rk.recv[r], i, a);
    }
}

// Largest message per rank that takes hb_twoshot_wave.
constexpr uint64_t kWaveTableMaxBytes = (uint64_t)16 << 20;

namespace {

template <typename T, int RMAX, bool EXACT, int U, bool NT, int NODE = 0>
hipError_t launch_one(const HBParams<RMAX> &p, uint32_t grid, uint32_t threads, hipStream_t stream)
{
    if constexpr (RMAX == 32 && U == 1) {
        if (p.nvec * 16 <= kWaveTableMaxBytes && threads % 64 == 0) {
            hipLaunchKernelGGL((hb_twoshot_wave<T, EXACT, NT, NODE>), dim3(grid), dim3(threads), 0,
                               stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((hb_twoshot<T, RMAX, EXACT, U, NT, NODE>), dim3(grid), dim3(threads), 0,
                       stream, p);
    return hipGetLastError();
}

// The hierarchical order, at one vector per lane.  Node sizes 2, 4, 8 and 16
// on the exact rank tables are compiled as constants; any other shape takes
// the node size at run time (same results, more instructions).
template <typename T, int RMAX, bool EXACT, bool NT>
hipError_t launch_grouped(const HBParams<RMAX> &p, uint32_t grid, uint32_t threads,
                          hipStream_t stream)
{
    if constexpr (EXACT) {
        if constexpr (RMAX > 2)
            if (p.group == 2)
                return launch_one<T, RMAX, true, 1, NT, 2>(p, grid, threads, stream);
        if constexpr (RMAX > 4)
            if (p.group == 4)
                return launch_one<T, RMAX, true, 1, NT, 4>(p, grid, threads, stream);
        if constexpr (RMAX > 8)
            if (p.group == 8)
                return launch_one<T, RMAX, true, 1, NT, 8>(p, grid, threads, stream);
        if constexpr (RMAX > 16)
            if (p.group == 16)
                return launch_one<T, RMAX, true, 1, NT, 16>(p, grid, threads, stream);
    }
    return launch_one<T, RMAX, EXACT, 1, NT, -1>(p, grid, threads, stream);
}

// Largest vectors-per-lane count compiled for a rank table size (register
// budget: U * RMAX * 4 VGPRs of loaded data per lane).
constexpr int max_unroll(int rmax) { return rmax <= 4 ? 4 : (rmax <= 8 ? 2 : 1); }

template <typename T, int RMAX, bool EXACT>
hipError_t launch_unroll(const HBParams<RMAX> &p, uint32_t grid, uint32_t threads, int u,
                         bool nt, hipStream_t stream)
{
    constexpr int kMax = max_unroll(RMAX);
    if (p.group != 0)
        return nt ? launch_grouped<T, RMAX, EXACT, true>(p, grid, threads, stream)
                  : launch_grouped<T, RMAX, EXACT, false>(p, grid, threads, stream);
    if (u >= 4 && kMax >= 4)
        return nt ? launch_one<T, RMAX, EXACT, (kMax >= 4 ? 4 : 1), true>(p, grid, threads, stream)
                  : launch_one<T, RMAX, EXACT, (kMax >= 4 ? 4 : 1), false>(p, grid, threads, stream);
    if (u >= 2 && kMax >= 2)
        return nt ? launch_one<T, RMAX, EXACT, (kMax >= 2 ? 2 : 1), true>(p, grid, threads, stream)
                  : launch_one<T, RMAX, EXACT, (kMax >= 2 ? 2 : 1), false>(p, grid, threads, stream);
    return nt ? launch_one<T, RMAX, EXACT, 1, true>(p, grid, threads, stream)
              : launch_one<T, RMAX, EXACT, 1, false>(p, grid, threads, stream);
}

template <typename T, int RMAX, bool EXACT>
hipError_t launch_table(const void *const *send, void *const *recv, size_t count, int nranks,
                        const HBConfig &cfg, int want_threads, uint64_t want_blocks, int group,
                        bool nt, hipStream_t stream)
{
    constexpr uint64_t kPerVec = 16 / T::kBytes;
    HBParams<RMAX> p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    p.nvec = count / kPerVec;
    p.tail_elems = (uint32_t)(count % kPerVec);
    p.chunk_vec = p.nvec / (uint64_t)nranks;
    p.nranks = (uint32_t)nranks;
    p.interleaved = cfg.interleaved ? 1u : 0u;
    p.group = group > 1 && group < nranks ? (uint32_t)group : 0u;

    int u = cfg.unroll > 0 ? cfg.unroll : 1;
    if (u > max_unroll(RMAX))
        u = max_unroll(RMAX);
    // Defaults: hb_default_threads threads and hb_default_blocks_per_cu
    // workgroups per CU (one for 6 to 8 and from 16 ranks: there, fewer loads
    // in flight per CU stream HBM faster; more for fewer ranks).
    uint32_t threads = want_threads > 0 ? (uint32_t)want_threads
                                        : (uint32_t)hb_default_threads(nranks, count * T::kBytes);
    if (threads > (uint32_t)hb_max_threads(RMAX))
        threads = (uint32_t)hb_max_threads(RMAX);
    const uint64_t blocks =
        want_blocks > 0 ? want_blocks
                        : (uint64_t)cfg.cu_count *
                              (uint64_t)hb_default_blocks_per_cu(nranks, count * T::kBytes);

    // Enough workgroups to fill the chip, but never more per chunk than the
    // largest chunk has tiles.
    const uint64_t tile = (uint64_t)threads * (uint64_t)u;
    const uint64_t largest = p.interleaved
                                 ? (p.nvec + (uint64_t)nranks - 1) / (uint64_t)nranks
                                 : p.nvec - p.chunk_vec * (uint64_t)(nranks - 1);
    const uint64_t tiles = (largest + tile - 1) / tile;
    // Workgroups per chunk rounded down: a grid just above a multiple of the
    // CU count would leave a few CUs with twice the work (R = 3 at one per
    // CU: 86 x 3 = 258 workgroups on 256 CUs).
    uint64_t want = blocks / (uint64_t)nranks;
    if (want < 1)
        want = 1;
    uint64_t bpc = tiles < want ? tiles : want;
    if (bpc < 1)
        bpc = 1;
    // A few more workgroups than that when they save a round of tiles while
    // each workgroup has few (12 ranks at 512 KiB per rank: 22 tiles per
    // chunk on 21 workgroups gave one of them a second tile); with many
    // rounds one more costs less than the uneven load of the extra groups.
    // At one workgroup per CU, two rounds become one with up to twice the
    // workgroups (16 ranks at 1 MiB per rank: 512 workgroups, 5.5 against
    // 6.6 us; 32 ranks 10.4 against 11.5 us); with more rounds, or more
    // workgroups per CU already, the extra groups weigh more.
    const uint64_t rounds = (tiles + bpc - 1) / bpc;
    if (want_blocks == 0 && rounds == 2 && tiles <= 2 * bpc &&
        blocks <= (uint64_t)cfg.cu_count) {
        bpc = tiles;
    } else if (want_blocks == 0 && rounds > 1 && rounds <= 4) {
        const uint64_t fewer = (tiles + rounds - 2) / (rounds - 1);
        if (fewer * (uint64_t)nranks * 4 <= blocks * 5)
            bpc = fewer;
    }
    p.blocks_per_chunk = (uint32_t)bpc;
    const uint32_t grid = (uint32_t)(bpc * (uint64_t)nranks);
    if (cfg.rec != nullptr)
        *cfg.rec = {arProtoHB, 1, grid, threads, 0, nt ? 1 : 0, (int32_t)p.group, 0};
    return launch_unroll<T, RMAX, EXACT>(p, grid, threads, u, nt, stream);
}

template <typename T>
hipError_t launch_dtype(const void *const *send, void *const *recv, size_t count, int nranks,
                        const HBConfig &cfg, int th, uint64_t bl, int grp, bool nt,
                        hipStream_t stream)
{
    switch (nranks) {
    case 1: return launch_table<T, 1, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    case 2: return launch_table<T, 2, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    case 4: return launch_table<T, 4, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    case 8: return launch_table<T, 8, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    case 16: return launch_table<T, 16, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    case 32: return launch_table<T, 32, true>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    default: break;
    }
    if (nranks < 4)
        return launch_table<T, 4, false>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    if (nranks < 8)
        return launch_table<T, 8, false>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    if (nranks < 16)
        return launch_table<T, 16, false>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
    return launch_table<T, 32, false>(send, recv, count, nranks, cfg, th, bl, grp, nt, stream);
}

}  // namespace

hipError_t launch_hb(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const HBConfig &cfg, int threads, uint64_t blocks, int group,
                     bool nt, hipStream_t stream)
{
    switch (dtype) {
    case kBf16:
        return launch_dtype<Bf16>(send, recv, count, nranks, cfg, threads, blocks, group, nt,
                                  stream);
    case kFp16:
        return launch_dtype<Fp16>(send, recv, count, nranks, cfg, threads, blocks, group, nt,
                                  stream);
    default:
        return launch_dtype<Fp32>(send, recv, count, nranks, cfg, threads, blocks, group, nt,
                                  stream);
    }
}

}  // namespace ar
