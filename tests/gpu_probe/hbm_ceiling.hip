// hbm_ceiling.hip -- measurement aid: the HB kernel's memory traffic without
// its arithmetic, to bound what the reduction itself costs.
//
// Eight rank streams of 16-byte vectors, walked with the same workgroup-to-
// tile mapping as the HB two-shot's default layout (workgroup w serves chunk
// w % 8; chunk c is every 8th tile of blockDim.x vectors starting at tile c),
// with the same non-temporal 128-bit loads and stores (but for mode 3).  Modes:
//   0 read   load the 8 streams, fold them with xor, and store one vector per
//            thread to `sink` at the end (grid * blockDim vectors in all);
//   1 write  store a vector derived from the index to the 8 streams;
//   2 copy   load the 8 streams and store them to dst[0..7] at the same
//            offset (dst == src: in place, the HB prefill's access pattern);
//   3 write  as mode 1, with ordinary (cached) stores instead of non-temporal.
// Not part of the library: built by __graft_entry__.build() next to the
// converter probe, checked by tests/test_gpu_probe_hbm.py, and timed by
// bench.py --only ceilings.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct CeilingParams {
    const u32x4 *src[8];
    u32x4 *dst[8];
    u32x4 *sink;
    uint64_t nvec;           // vectors per stream
    uint32_t blocks_per_chunk;
    int mode;
};

__global__ __launch_bounds__(1024) void hbm_ceiling(CeilingParams p)
{
    const uint64_t tile = blockDim.x;
    const uint32_t c = blockIdx.x % 8u;
    const uint32_t bb = blockIdx.x / 8u;
    const uint64_t start = ((uint64_t)bb * 8u + c) * tile;
    const uint64_t step = (uint64_t)p.blocks_per_chunk * 8u * tile;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t base = start; base < p.nvec; base += step) {
        const uint64_t i = base + threadIdx.x;
        if (i >= p.nvec)
            continue;
        if (p.mode == 1 || p.mode == 3) {
            const u32x4 v = {(uint32_t)i, (uint32_t)(i >> 32), c, 0x9e3779b9u};
            if (p.mode == 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    __builtin_nontemporal_store(v, p.dst[j] + i);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    p.dst[j][i] = v;
            }
            continue;
        }
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = __builtin_nontemporal_load(p.src[j] + i);
        if (p.mode == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc ^= v[j];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                __builtin_nontemporal_store(v[j], p.dst[j] + i);
        }
    }
    if (p.mode == 0)
        p.sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// grid must be a positive multiple of 8 and threads a multiple of 64 in
// 64..1024; sink must hold grid * threads vectors for mode 0.  Returns 0, or
// -1 for a bad launch shape or a launch error.
extern "C" int hbm_ceiling_run(void *const *src, void *const *dst, void *sink, uint64_t nvec,
                               int mode, int grid, int threads, void *stream)
{
    if (grid < 8 || grid % 8 != 0 || threads < 64 || threads > 1024 || threads % 64 != 0 ||
        mode < 0 || mode > 3)
        return -1;
    CeilingParams p;
    for (int j = 0; j < 8; ++j) {
        p.src[j] = (const u32x4 *)src[j];
        p.dst[j] = (u32x4 *)dst[j];
    }
    p.sink = (u32x4 *)sink;
    p.nvec = nvec;
    p.blocks_per_chunk = (uint32_t)(grid / 8);
    p.mode = mode;
    hipLaunchKernelGGL(hbm_ceiling, dim3((uint32_t)grid), dim3((uint32_t)threads), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
