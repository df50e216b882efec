// hbm_ceiling.hip -- measurement aid: the HB kernel's memory traffic without
// its arithmetic, to bound what the reduction itself costs.
//
// S rank streams of 16-byte vectors (S = 8, 16 or 32: the rank counts of the
// configured workloads), walked with the same workgroup-to-tile mapping as
// the HB two-shot's default layout (workgroup w serves chunk w % S; chunk c
// is every S-th tile of blockDim.x vectors starting at tile c), with the same
// non-temporal 128-bit loads and stores (but for mode 3).  Modes:
//   0 read   load the S streams, fold them with xor, and store one vector per
//            thread to `sink` at the end (grid * blockDim vectors in all);
//   1 write  store a vector derived from the index to the S streams;
//   2 copy   load the S streams and store them to dst[0..S-1] at the same
//            offset (dst == src: in place, the HB prefill's access pattern;
//            dst != src: out of place, 2 * S streams, as HB at R = S);
//   3 write  as mode 1, with ordinary (cached) stores instead of non-temporal.
// Not part of the library: built by __graft_entry__.build() next to the
// converter probe, checked by tests/test_gpu_probe_hbm.py, and timed by
// bench.py (the hbm_ceilings fields).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int S>
struct CeilingParams {
    const u32x4 *src[S];
    u32x4 *dst[S];
    u32x4 *sink;
    uint64_t nvec;           // vectors per stream
    uint32_t blocks_per_chunk;
    int mode;
};

// Largest workgroup per stream count: the S vectors a lane holds (4 VGPRs
// each) must fit its register share without spilling, as in the HB kernel.
constexpr int ceiling_max_threads(int s) { return s >= 32 ? 256 : (s >= 16 ? 512 : 1024); }

template <int S>
__global__ __launch_bounds__(ceiling_max_threads(S)) void hbm_ceiling(CeilingParams<S> p)
{
    const uint64_t tile = blockDim.x;
    const uint32_t c = blockIdx.x % (uint32_t)S;
    const uint32_t bb = blockIdx.x / (uint32_t)S;
    const uint64_t start = ((uint64_t)bb * S + c) * tile;
    const uint64_t step = (uint64_t)p.blocks_per_chunk * S * tile;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t base = start; base < p.nvec; base += step) {
        const uint64_t i = base + threadIdx.x;
        if (i >= p.nvec)
            continue;
        if (p.mode == 1 || p.mode == 3) {
            const u32x4 v = {(uint32_t)i, (uint32_t)(i >> 32), c, 0x9e3779b9u};
            if (p.mode == 1) {
#pragma unroll
                for (int j = 0; j < S; ++j)
                    __builtin_nontemporal_store(v, p.dst[j] + i);
            } else {
#pragma unroll
                for (int j = 0; j < S; ++j)
                    p.dst[j][i] = v;
            }
            continue;
        }
        u32x4 v[S];
#pragma unroll
        for (int j = 0; j < S; ++j)
            v[j] = __builtin_nontemporal_load(p.src[j] + i);
        if (p.mode == 0) {
#pragma unroll
            for (int j = 0; j < S; ++j)
                acc ^= v[j];
        } else {
#pragma unroll
            for (int j = 0; j < S; ++j)
                __builtin_nontemporal_store(v[j], p.dst[j] + i);
        }
    }
    if (p.mode == 0)
        p.sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int S>
static int run(void *const *src, void *const *dst, void *sink, uint64_t nvec, int mode, int grid,
               int threads, void *stream)
{
    CeilingParams<S> p;
    for (int j = 0; j < S; ++j) {
        p.src[j] = (const u32x4 *)src[j];
        p.dst[j] = (u32x4 *)dst[j];
    }
    p.sink = (u32x4 *)sink;
    p.nvec = nvec;
    p.blocks_per_chunk = (uint32_t)(grid / S);
    p.mode = mode;
    hipLaunchKernelGGL((hbm_ceiling<S>), dim3((uint32_t)grid), dim3((uint32_t)threads), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `nstreams` S is 8, 16 or 32 (src and dst each hold S pointers); grid must
// be a positive multiple of S and threads a multiple of 64 from 64 up to
// 1024 (8 streams), 512 (16) or 256 (32); sink must hold grid * threads
// vectors for mode 0.  Returns 0, or -1 for a bad stream count or launch
// shape, or a launch error.
extern "C" int hbm_ceiling_run_n(void *const *src, void *const *dst, void *sink, uint64_t nvec,
                                 int mode, int grid, int threads, int nstreams, void *stream)
{
    if ((nstreams != 8 && nstreams != 16 && nstreams != 32) || grid < nstreams ||
        grid % nstreams != 0 || threads < 64 || threads > ceiling_max_threads(nstreams) ||
        threads % 64 != 0 || mode < 0 || mode > 3)
        return -1;
    switch (nstreams) {
    case 8: return run<8>(src, dst, sink, nvec, mode, grid, threads, stream);
    case 16: return run<16>(src, dst, sink, nvec, mode, grid, threads, stream);
    default: return run<32>(src, dst, sink, nvec, mode, grid, threads, stream);
    }
}

// The 8-stream form (the R = 8 prefill's shape).
extern "C" int hbm_ceiling_run(void *const *src, void *const *dst, void *sink, uint64_t nvec,
                               int mode, int grid, int threads, void *stream)
{
    return hbm_ceiling_run_n(src, dst, sink, nvec, mode, grid, threads, 8, stream);
}
