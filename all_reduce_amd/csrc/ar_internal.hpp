// ar_internal.hpp -- what the C ABI layer and the kernel files share.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ar_allreduce.h"

namespace ar {

enum DType { kBf16 = 0, kFp16 = 1, kFp32 = 2 };

// Occupancy-derived cap on co-resident LL workgroups: LL consumers wait on
// packets from other workgroups, so every workgroup of an LL grid must be
// resident at once.  Indexed [dtype][rank variant][thread-count index].
constexpr int kRankVariants = 6;  // 1, 2, 4, 8, 16, 32 -> exact kernels; others -> generic
constexpr int kThreadChoices = 5; // 64, 128, 256, 512, 1024

// Default LL launch shape for a call that names none and has no tuned entry:
// threads per workgroup and workgroups per rank, by rank count (up to 4, 5-8,
// 9-16, 17-32) and message size per rank, for 8-byte packets.  Each entry is
// the fastest of a grid measured on MI355X (bf16, graph-replayed calls,
// 64-1024 threads, 1-128 workgroups per rank) at a power-of-two size from
// 2 KiB to 1 MiB per rank, or one within measurement noise of it that is also
// the best at a neighbouring size.  A size takes the entry of the next power
// of two up, and sizes above 1 MiB the last one.  The first two rows differ
// at 256 and 512 KiB, where up to 4 ranks word packets run with 512 x 64
// (bf16 at 2 ranks, 512 KiB: 3.85 against 4.86 us with 512 x 32; 4 ranks
// 4.33 against 4.91) and at 8 ranks (fp32) 256 x 32 and 512 x 32 lead.
struct LLShape {
    int threads;
    int per_rank;
};

inline LLShape ll_default_shape(int nranks, uint64_t bytes_per_rank)
{
    static constexpr LLShape kTable[4][10] = {
        // 2K        4K        8K        16K       32K        64K
        // 128K      256K       512K       1M
        {{256, 1}, {256, 2}, {256, 4}, {256, 8}, {256, 16}, {256, 64},
         {256, 64}, {512, 64}, {512, 64}, {512, 32}},
        {{256, 1}, {256, 2}, {256, 4}, {256, 8}, {256, 16}, {256, 64},
         {256, 64}, {256, 32}, {512, 32}, {512, 32}},
        {{512, 1}, {512, 1}, {512, 2}, {512, 4}, {256, 8}, {256, 32},
         {256, 64}, {128, 128}, {512, 16}, {512, 16}},
        {{512, 1}, {512, 1}, {512, 1}, {512, 2}, {512, 4}, {512, 16},
         {256, 16}, {128, 32}, {512, 8}, {512, 8}},
    };
    int s = 0;
    while (s < 9 && ((uint64_t)2048 << s) < bytes_per_rank)
        ++s;
    return kTable[nranks <= 4 ? 0 : (nranks <= 8 ? 1 : (nranks <= 16 ? 2 : 3))][s];
}

// The same for the three-element packets of bfloat16 and float16 (ll_dense.hip),
// from the size per rank where they are the default packet (ll_dense_from_bytes;
// below it the entries are unused): measured on MI355X like the word table,
// 64-512 threads, 1-128 workgroups per rank (the occupancy cap applies).
inline LLShape ll_dense_default_shape(int nranks, uint64_t bytes_per_rank)
{
    static constexpr LLShape kTable[3][10] = {
        // 2K        4K        8K        16K       32K        64K
        // 128K      256K       512K       1M
        {{256, 1}, {256, 2}, {256, 4}, {256, 8}, {256, 16}, {256, 32},
         {256, 64}, {64, 128}, {256, 64}, {256, 128}},
        {{512, 1}, {512, 1}, {512, 2}, {512, 4}, {256, 8}, {256, 32},
         {256, 32}, {256, 128}, {128, 128}, {128, 64}},
        {{512, 1}, {512, 1}, {512, 1}, {512, 2}, {512, 4}, {512, 8},
         {256, 16}, {128, 128}, {128, 128}, {512, 64}},
    };
    int s = 0;
    while (s < 9 && ((uint64_t)2048 << s) < bytes_per_rank)
        ++s;
    return kTable[nranks <= 8 ? 0 : (nranks <= 16 ? 1 : 2)][s];
}

// Bytes per rank from which three-element packets are the default: measured
// on MI355X, they cost about 0.5 us of LDS staging per call at small sizes and
// win from 256 KiB per rank at 8 ranks (1 MiB: 7.95 against 9.79 us; 192 KiB
// still goes to word packets, 4.05 against 4.23 us) and at the generic counts
// 3, 5, 6 and 7, above 512 KiB at 1, 2 and 4 ranks (2 ranks: word 4.8 against
// 6.6 us at 512 KiB, three-element 5.4 against 5.6 us at 640 KiB), above
// 128 KiB at 9 to 16 ranks (128 KiB: word 4.6 against 4.9 us at 16 ranks;
// 136 KiB: 5.2 against 6.3 us) and from 128 KiB above 16 (1 MiB at 32: 28.5
// against 37.7 us).
inline uint64_t ll_dense_from_bytes(int nranks)
{
    if (nranks == 1 || nranks == 2 || nranks == 4)
        return ((uint64_t)512 << 10) + 1;
    if (nranks <= 8)
        return (uint64_t)256 << 10;
    return nranks <= 16 ? ((uint64_t)128 << 10) + 1 : ((uint64_t)128 << 10);
}

// Default threads per workgroup of the fused HB kernel (one workgroup per
// CU), by rank count and message size per rank, measured on MI355X: 256 up to
// 8 ranks; from 9 to 16 ranks 128 up to 16 MiB per rank (2^18 fp16 at 16
// ranks: 4.2 against 5.1 us with 256) and 64 above (4096 x 7168 fp32: 671
// against 689 us); 128 from 17 ranks.
inline int hb_default_threads(int nranks, uint64_t bytes_per_rank)
{
    if (nranks <= 8)
        return 256;
    if (nranks <= 16)
        return bytes_per_rank <= ((uint64_t)16 << 20) ? 128 : 64;
    return 128;
}

// Default workgroups per CU of the fused HB kernel.  Each lane holds one
// 16-byte vector per rank in flight, so with few ranks one workgroup per CU
// leaves HBM idle: measured on MI355X (bf16, 4-128 MiB per rank, in place and
// out of place), the fastest point keeps about 2048 loads in flight per CU
// for 256-thread workgroups -- 8 workgroups per CU at 1 rank (44 against
// 131 us at 128 MiB), 4 at 2, 3 at 3, 2 at 4 and 5, 1 from 6 -- and 4 (2 up
// to 16 MiB per rank) for 9 to 15 ranks, whose default is 64 threads above
// 16 MiB (12 ranks, 128 MiB: 587-620 against 1172 us).  Below 4 MiB per rank
// and at 8, 16 and from 17 ranks, one.
inline int hb_default_blocks_per_cu(int nranks, uint64_t bytes_per_rank)
{
    if (bytes_per_rank < ((uint64_t)4 << 20))
        return 1;
    if (nranks <= 5) {
        static constexpr int kPerCU[6] = {1, 8, 4, 3, 2, 2};
        return kPerCU[nranks < 0 ? 0 : nranks];
    }
    if (nranks >= 9 && nranks <= 15)
        return bytes_per_rank > ((uint64_t)16 << 20) ? 4 : 2;
    return 1;
}

// LL flag schemes (the values of arOptLLFlagScheme): the reader zeroes each
// consumed packet (the default), or each 512-byte packet group carries a
// sequence number.
constexpr int kSchemeCleared = 0;
constexpr int kSchemeSequenced = 1;

// LL node layouts (the kernels' NODE parameter): the flat order, nodes
// marked by a run-time bitmask (any node size), or nodes of a compile-time
// size (2, 4, 8 or 16 ranks; a power-of-two rank count admits no other).
constexpr int kNodeFlat = 0;
constexpr int kNodeMask = -1;

// LL kernel kinds with their own occupancy: the cleared scheme in the flat
// order, the sequenced scheme (flat order only), then the cleared scheme in
// the hierarchical order with a node bitmask, or with nodes of 2, 4, 8 or 16,
// and last the three-element packets (ll_dense.hip; 16-bit types, flat order,
// cleared scheme, packet-width index 0).
constexpr int kLLKinds = 8;
constexpr int kLLDenseKind = 7;
constexpr int ll_kind(bool seq, int node)
{
    return node == kNodeFlat ? (seq ? 1 : 0)
         : node == kNodeMask ? 2
         : node == 2 ? 3 : node == 4 ? 4 : node == 8 ? 5 : 6;
}

}  // namespace ar

constexpr int kOptionCount = 16;

namespace ar {
// One tuned launch shape: threads per workgroup and workgroups (HB: the
// whole grid; LL: per simulated rank), with the time it measured.  0 threads
// and 0 blocks mean the built-in default shape won.  valid == 0: not tuned.
struct TunedShape {
    int32_t valid;
    int32_t threads;
    int32_t blocks;
    int32_t pkt_bytes;  // LL packet width it was timed with: 8 (HB: 0)
    int32_t nt;         // HB: non-temporal (1) or cached (0) accesses won (LL: 0)
    float us;
};
// Message sizes are bucketed by ceil(log2(bytes per rank)).
constexpr int kBuckets = 41;

// What the communicator's most recent launch was (arCommGetLastLaunch).
struct LaunchRecord {
    int32_t protocol;   // arProtoLL or arProtoHB; -1 before the first launch
    int32_t kernels;    // kernels enqueued by the call
    uint32_t grid;      // workgroups of the (first) kernel
    uint32_t threads;   // threads per workgroup
    int32_t pkt_bytes;  // LL packet width (HB: 0)
    int32_t nt;         // HB: non-temporal accesses (LL: 0)
    int32_t node;       // ranks per node of a hierarchical order, else 0
    int32_t staged;     // HB: 1 for a staged form (kernel boundary between shots)
    int32_t payload;    // LL payload bytes per packet: 4 and 8 (word packets of 8 and
                        // 16 bytes), 6 (three 16-bit elements); HB: 0
};
}  // namespace ar

struct arComm {
    int device;
    int max_ranks;
    size_t max_ll_bytes;
    int cu_count;
    uint64_t wall_clock_khz;
    uint64_t *pkts;        // 2 * max_ranks * max_ll_bytes bytes, rounded up
    uint64_t pkt_stride;   // 8-byte packets per rank region, a multiple of 64 (512 bytes)
    uint32_t *seq;         // sequence table: one entry per 512-byte group and rank region
    uint64_t seq_words;    // (pkt_stride / 64) * max_ranks
    uint32_t *ctrl;        // control words; [0] is the async error
    int64_t opt[kOptionCount]; // indexed by arOption_t
    // [kernel kind (ar::ll_kind)][packet width: 8 B, 16 B][dtype]
    // [rank variant][thread-count index]
    int ll_resident[ar::kLLKinds][2][3][ar::kRankVariants + 1][ar::kThreadChoices];
    bool ll16_ok;          // the packet scratch is small enough for 16-byte packets
    // [dtype][nranks][protocol][in place][bucket]; filled by arCommTune.  In
    // place and out of place are tuned apart: on MI355X they favour different
    // shapes (8 x 128 MiB bf16: 256 x 256 is fastest in place, 512 workgroups
    // out of place, each about 10 % off on the other).
    ar::TunedShape tuned[3][AR_MAX_RANKS + 1][2][2][ar::kBuckets];
    // Written by the launchers (which see the communicator as const): the
    // shape of the most recent launch, for arCommGetLastLaunch.
    mutable ar::LaunchRecord last;
    // Caller-owned device memory for the staged two-level HB form's node
    // partials (arCommSetWorkspace); nullptr: none.
    void *ws;
    size_t ws_bytes;
};

namespace ar {

// What the HB launchers need besides the call's arguments: the chip's compute
// units (the default grid), the vectors per lane and the chunk layout, and
// where to record the launch (may be null).  Built from a communicator's
// options, or from the defaults by the entry point that has none.
struct HBConfig {
    int cu_count;
    int unroll;          // 16-byte vectors per lane per rank (0: 1)
    bool interleaved;    // chunk c = every R-th tile (else contiguous N/R)
    LaunchRecord *rec;
};

// Launchers: validate nothing (the ABI layer did), pick the instantiation,
// enqueue on `stream`.  `threads` and `blocks` give the launch shape (HB: the
// whole grid; LL: workgroups per rank); 0 picks the built-in default.  Both
// are clamped to what the kernel and the message allow.  Return hipSuccess or
// the launch error.
// `group` > 0 selects the hierarchical summation order (groups of `group`
// consecutive ranks first, then the group partials); the caller guarantees
// 1 < group < nranks and nranks % group == 0.  `nt` selects non-temporal
// loads and stores (else ordinary, cached ones).
hipError_t launch_hb(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const HBConfig &cfg, int threads, uint64_t blocks, int group,
                     bool nt, hipStream_t stream);
// `pkt_bytes` 16 selects 16-byte LL packets (the caller checks comm->ll16_ok),
// anything else 8-byte packets; `scheme` kSchemeSequenced the sequenced flag
// scheme, anything else the cleared one.  `group` as for launch_hb; the caller
// never combines it with the sequenced scheme.
hipError_t launch_ll(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const arComm *comm, int threads, uint64_t blocks, int pkt_bytes,
                     int scheme, int group, hipStream_t stream);
// The staged form of the HB two-shot (reduce-scatter into the owner's output,
// kernel boundary, all-gather from it), flat order only.
hipError_t launch_hb_staged(const void *const *send, void *const *recv, size_t count, int dtype,
                            int nranks, const HBConfig &cfg, int threads, uint64_t blocks, bool nt,
                            hipStream_t stream);
// The staged two-level form for nranks = G * group ranks in G nodes of
// `group` (1 < group < nranks, group divides nranks): stage 1 writes each
// node's binary32 partial to `ws` (node g at ws + g * hier_partial_stride),
// a kernel boundary, stage 2 folds the G partials in node order, rounds once
// and writes every output.  The caller checks that `ws` holds
// hier_workspace_bytes(count, nranks / group) bytes, 256-byte aligned.
hipError_t launch_hb_hier(const void *const *send, void *const *recv, size_t count, int dtype,
                          int nranks, int group, void *ws, const HBConfig &cfg, int threads,
                          uint64_t blocks, bool nt, hipStream_t stream);
// Bytes between two nodes' partials, and the workspace the two-level form
// needs: one binary32 per element per node, each node's share rounded up to
// 256 bytes.  The workspace size saturates at UINT64_MAX instead of wrapping
// (no message that passes argument validation comes near it), so a size
// check against it can only refuse.
inline uint64_t hier_partial_stride(uint64_t count) { return (count * 4 + 255) / 256 * 256; }
inline uint64_t hier_workspace_bytes(uint64_t count, int nodes)
{
    if (nodes <= 0)
        return 0;
    if (count > (UINT64_MAX - 255) / 4)
        return UINT64_MAX;
    const uint64_t stride = hier_partial_stride(count);
    return stride > UINT64_MAX / (uint64_t)nodes ? UINT64_MAX : stride * (uint64_t)nodes;
}
// The LL one-shot with three-element packets (bfloat16 / float16 only, flat
// order, cleared scheme, 8-byte packets).
hipError_t launch_ll_dense(const void *const *send, void *const *recv, size_t count, int dtype,
                           int nranks, const arComm *comm, int threads, uint64_t blocks,
                           hipStream_t stream);
// Its occupancy table, [dtype][rank variant][thread-count index].
hipError_t query_ll_dense_residency(int (*per_cu)[kRankVariants + 1][kThreadChoices]);
// Zeroes the packets and the error word and sets the sequence table to
// arOptDebugSeqStart (0 by default).
hipError_t launch_reset(const arComm *comm, hipStream_t stream);
// Fills comm->ll_resident from the occupancy calculator.
hipError_t query_ll_residency(arComm *comm);

}  // namespace ar
