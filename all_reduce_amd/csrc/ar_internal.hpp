// ar_internal.hpp -- what the C ABI layer and the kernel files share.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ar_allreduce.h"

namespace ar {

// Rank pointer table, passed by value in the kernel arguments: the host-built
// "channels" of the simulated group (the microsoft/mscclpp project summary,
// agentlenshq.com, "How it works": channels are set up on the host and used
// from device code).  Sized for the kernel's compile-time rank count.
template <int R>
struct RankTable {
    const void *send[R];
    void *recv[R];
};

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

// One-shot LL launch parameters.
template <int R>
struct LLParams {
    RankTable<R> rk;
    uint64_t *pkts;          // packet scratch; rank k's packets start at k * pkt_stride
    uint64_t pkt_stride;
    uint64_t npkt;           // packets per rank = ceil(bytes per rank / 4)
    uint64_t put_per_block;  // packets each workgroup publishes for its rank
    uint64_t get_per_block;  // packets each workgroup polls, reduces and writes out
    uint32_t *ctrl;          // [0] async error (0 or arTimeout)
    uint64_t timeout_ticks;  // wall-clock ticks one packet wait may take
    uint32_t flag_skew;      // test hook: consumers wait for flag + skew
    uint32_t half_tail;      // 1 when the last packet carries only 2 payload bytes
    uint32_t nranks;
    uint32_t blocks_per_rank;
};

enum DType { kBf16 = 0, kFp16 = 1, kFp32 = 2 };

// Occupancy-derived cap on co-resident LL workgroups: LL consumers wait on
// packets from other workgroups, so every workgroup of an LL grid must be
// resident at once.  Indexed [dtype][rank variant][thread-count index].
constexpr int kRankVariants = 6;  // 1, 2, 4, 8, 16, 32 -> exact kernels; others -> generic
constexpr int kThreadChoices = 5; // 64, 128, 256, 512, 1024

}  // namespace ar

constexpr int kOptionCount = 10;

namespace ar {
// One tuned launch shape: threads per workgroup and workgroups (HB: the
// whole grid; LL: per simulated rank), with the time it measured.  0 threads
// and 0 blocks mean the built-in default shape won.  valid == 0: not tuned.
struct TunedShape {
    int32_t valid;
    int32_t threads;
    int32_t blocks;
    float us;
};
// Message sizes are bucketed by ceil(log2(bytes per rank)).
constexpr int kBuckets = 41;
}  // namespace ar

struct arComm {
    int device;
    int max_ranks;
    size_t max_ll_bytes;
    int cu_count;
    uint64_t wall_clock_khz;
    uint64_t *pkts;        // 2 * max_ranks * max_ll_bytes bytes
    uint64_t pkt_stride;   // packets per rank region
    uint32_t *ctrl;        // control words; [0] is the async error
    int64_t opt[kOptionCount]; // indexed by arOption_t
    int ll_resident[3][ar::kRankVariants + 1][ar::kThreadChoices];
    // [dtype][nranks][protocol][bucket]; filled by arCommTune
    ar::TunedShape tuned[3][AR_MAX_RANKS + 1][2][ar::kBuckets];
};

namespace ar {

// Launchers: validate nothing (the ABI layer did), pick the instantiation,
// enqueue on `stream`.  `threads` and `blocks` give the launch shape (HB: the
// whole grid; LL: workgroups per rank); 0 picks the built-in default.  Both
// are clamped to what the kernel and the message allow.  Return hipSuccess or
// the launch error.
// `group` > 0 selects the hierarchical summation order (groups of `group`
// consecutive ranks first, then the group partials); the caller guarantees
// 1 < group < nranks and nranks % group == 0.
hipError_t launch_hb(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const arComm *comm, int threads, uint64_t blocks, int group,
                     hipStream_t stream);
hipError_t launch_ll(const void *const *send, void *const *recv, size_t count, int dtype,
                     int nranks, const arComm *comm, int threads, uint64_t blocks,
                     hipStream_t stream);
hipError_t launch_reset(const arComm *comm, hipStream_t stream);
// Fills comm->ll_resident from the occupancy calculator.
hipError_t query_ll_residency(arComm *comm);

}  // namespace ar
