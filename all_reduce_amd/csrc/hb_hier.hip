// hb_hier.hip -- the staged two-level HB all-reduce: node partials, a stage
// boundary, then a fold across nodes.
//
// The multi-node algorithms of SGLang's MSCCL++ integration for TP = 16 / 32
// ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南", blog.gitcode.com,
// section 4.4), and the high-throughput mode of NCCL EP, which moves data
// inside a node first and between nodes second ("NCCL EP统一MoE通信生态：打破
// 碎片化，加速大模型推理新纪元", itsolotime.com/archives/27456, section 3.2),
// reduce in two levels.  With R = G * L ranks in G nodes of L consecutive
// ranks:
//   stage 1  node-local reduce-scatter: for every position, node g's partial
//            is the binary32 sum of its L ranks in rank order (rank (g, c)
//            owns the c-th of the node's chunks; on one GPU ownership only
//            decides which workgroup does the work), written to node g's
//            partial vector in a workspace;
//   (the kernel boundary is the synchronisation between the levels: every
//    partial is complete before any is read)
//   stage 2  the exchange between nodes and the node-local all-gather: for
//            every position, the G node partials are summed in node order,
//            starting from node 0's exactly, rounded once to the element
//            type, and stored to all R outputs.
// Across real nodes, stage 2 would ship each chunk's partial to the G - 1
// peer ranks of the same local index (1 / L of the message per link) and
// all-gather inside the node; here the G partials are read from the
// workspace once per position and the result is written to every rank, as
// the one-GPU LL and HB kernels reduce each element once.
//
// The partials stay in binary32 and are rounded once (the two-level order's
// reading; a real deployment would usually ship them in the element type and
// round twice).  The result equals that of the fused HB kernel in the same
// hierarchical order, bit for bit.
//
// Traffic: stage 1 reads R * N * s bytes and writes G * N * 4; stage 2 reads
// G * N * 4 and writes R * N * s.  So 2 * G * N * 4 bytes more than the fused
// kernel: +1/8 for fp32 at R = 32 in nodes of 8, +1/4 for fp16 at R = 16 in
// nodes of 8.  In place is safe: stage 1 only reads the inputs and stage 2,
// which writes the outputs, never reads them.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

struct HierParams {
    RankTable<AR_MAX_RANKS> rk;
    float *ws;            // node g's partials start at ws + g * pstride
    uint64_t pstride;     // floats between two nodes' partials (a multiple of 64)
    uint64_t nvec;        // whole 16-byte vectors per rank
    uint32_t nranks;
    uint32_t node;        // ranks per node, L
    uint32_t nodes;       // nodes, G
    uint32_t tail_elems;  // elements after the last whole vector
};

constexpr int kHierMaxThreads = 512;

// Elements per 16-byte vector of the element type, and the partial floats of
// one vector: 8 for the 16-bit types (two 16-byte partial vectors), 4 for fp32.
template <typename T>
constexpr int per_vec() { return 16 / T::kBytes; }

__device__ inline float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }

template <typename T>
__device__ inline float tail_load(const void *base, uint64_t i)
{
    uint32_t w = (T::kBytes == 2) ? (uint32_t)((const uint16_t *)base)[i]
                                  : ((const uint32_t *)base)[i];
    float f[T::kPerWord];
    T::widen(w, f);
    return f[0];
}

template <typename T>
__device__ inline void tail_store(void *base, uint64_t i, float a)
{
    float f[T::kPerWord] = {};
    f[0] = a;
    const uint32_t w = T::narrow(f);
    if constexpr (T::kBytes == 2)
        ((uint16_t *)base)[i] = (uint16_t)w;
    else
        ((uint32_t *)base)[i] = w;
}

// Stage 1.  LC: ranks per node at compile time (2, 4, 8 or 16), or 0 for any
// node size up to 16 read from p.node.  Work items are (node, tile) pairs,
// nodes fastest, so consecutive workgroups stream different nodes' buffers at
// the same addresses.
template <typename T, int LC, bool NT>
__global__ __launch_bounds__(kHierMaxThreads) void hb_hier_partial(HierParams p)
{
    constexpr int LMAX = LC > 0 ? LC : 16;
    constexpr int PV = per_vec<T>();
    const uint32_t L = LC > 0 ? (uint32_t)LC : p.node;
    const uint64_t nthr = blockDim.x;
    const uint64_t items = (uint64_t)p.nodes * ((p.nvec + nthr - 1) / nthr);
    for (uint64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const uint32_t g = (uint32_t)(it % p.nodes);
        const uint64_t i = (it / p.nodes) * nthr + threadIdx.x;
        if (i >= p.nvec)
            continue;
        u32x4 v[LMAX];
#pragma unroll
        for (int j = 0; j < LMAX; ++j)
            if (LC > 0 || j < (int)L)
                v[j] = load16<NT>((const u32x4 *)p.rk.send[g * L + j] + i);
        float acc[PV];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            T::widen(v[0][q], acc + q * T::kPerWord);
#pragma unroll
        for (int j = 1; j < LMAX; ++j) {
            if (LC > 0 || j < (int)L) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float x[T::kPerWord];
                    T::widen(v[j][q], x);
#pragma unroll
                    for (int e = 0; e < T::kPerWord; ++e)
                        acc[q * T::kPerWord + e] = acc[q * T::kPerWord + e] + x[e];
                }
            }
        }
        u32x4 *dst = (u32x4 *)(p.ws + g * p.pstride + i * PV);
#pragma unroll
        for (int h = 0; h < PV / 4; ++h) {
            const u32x4 w = {__builtin_bit_cast(uint32_t, acc[4 * h]),
                             __builtin_bit_cast(uint32_t, acc[4 * h + 1]),
                             __builtin_bit_cast(uint32_t, acc[4 * h + 2]),
                             __builtin_bit_cast(uint32_t, acc[4 * h + 3])};
            store16<NT>(dst + h, w);
        }
    }

    // Elements after the last whole vector: the last workgroup, one lane per
    // (node, element).
    if (p.tail_elems != 0 && blockIdx.x == gridDim.x - 1) {
        for (uint32_t t = threadIdx.x; t < p.tail_elems * p.nodes; t += blockDim.x) {
            const uint32_t g = t / p.tail_elems;
            const uint64_t i = p.nvec * PV + t % p.tail_elems;
            float a = tail_load<T>(p.rk.send[g * L], i);
            for (uint32_t j = 1; j < L; ++j)
                a = a + tail_load<T>(p.rk.send[g * L + j], i);
            p.ws[g * p.pstride + i] = a;
        }
    }
}

// Stage 2.  GC: nodes at compile time (2, 4, 8 or 16), or 0 for any count up
// to 16 read from p.nodes.
template <typename T, int GC, bool NT>
__global__ __launch_bounds__(kHierMaxThreads) void hb_hier_fold(HierParams p)
{
    constexpr int GMAX = GC > 0 ? GC : 16;
    constexpr int PV = per_vec<T>();
    constexpr int H = PV / 4;  // 16-byte partial vectors per output vector
    const uint32_t G = GC > 0 ? (uint32_t)GC : p.nodes;
    const uint32_t n = p.nranks;
    const uint64_t nthr = blockDim.x;
    // The 32 output pointers come from a wave-held copy (WaveTable), and the
    // rank and node counts are re-read each iteration: kept in scalar
    // registers across the loop they spilled (48-167 lane writes per
    // instance; stage 2 at 16 x 112 MiB fp32 ran 438 us, now 405-409 us).
    WaveTable<AR_MAX_RANKS> wt(p.rk);
    for (uint64_t i = (uint64_t)blockIdx.x * nthr + threadIdx.x; i < p.nvec;
         i += (uint64_t)gridDim.x * nthr) {
        wt.refresh();
        uint32_t nl = n, Gl = G;
        asm volatile("" : "+s"(nl));
        if constexpr (GC == 0)
            asm volatile("" : "+s"(Gl));
        u32x4 pv[GMAX][H];
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
            if (GC > 0 || g < (int)Gl)
#pragma unroll
                for (int h = 0; h < H; ++h)
                    pv[g][h] = load16<NT>((const u32x4 *)(p.ws + g * p.pstride + i * PV) + h);
        // (each vector element goes through a uint32_t value before the bit
        // cast: hipcc bit-casts an element of a vector-typed lvalue wrongly,
        // reading another lane)
        float total[PV];
#pragma unroll
        for (int e = 0; e < PV; ++e)
            total[e] = as_float(pv[0][e / 4][e % 4]);
#pragma unroll
        for (int g = 1; g < GMAX; ++g)
            if (GC > 0 || g < (int)Gl)
#pragma unroll
                for (int e = 0; e < PV; ++e)
                    total[e] = total[e] + as_float(pv[g][e / 4][e % 4]);
        u32x4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            y[q] = T::narrow(total + q * T::kPerWord);
#pragma unroll
        for (int r = 0; r < AR_MAX_RANKS; ++r)
            if (r < (int)nl)
                store16<NT>((u32x4 *)wt.recv(r) + i, y);
    }

    if (p.tail_elems != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < p.tail_elems) {
        const uint64_t i = p.nvec * PV + threadIdx.x;
        float a = p.ws[i];
        for (uint32_t g = 1; g < G; ++g)
            a = a + p.ws[g * p.pstride + i];
        for (uint32_t r = 0; r < n; ++r)
            tail_store<T>(p.rk.recv[r], i, a);
    }
}

namespace {

template <typename T, int LC, bool NT>
hipError_t launch_partial(const HierParams &p, uint32_t grid, uint32_t threads, hipStream_t s)
{
    hipLaunchKernelGGL((hb_hier_partial<T, LC, NT>), dim3(grid), dim3(threads), 0, s, p);
    return hipGetLastError();
}

template <typename T, int GC, bool NT>
hipError_t launch_fold(const HierParams &p, uint32_t grid, uint32_t threads, hipStream_t s)
{
    hipLaunchKernelGGL((hb_hier_fold<T, GC, NT>), dim3(grid), dim3(threads), 0, s, p);
    return hipGetLastError();
}

template <typename T, bool NT>
hipError_t launch_stages(const HierParams &p, uint32_t grid1, uint32_t grid2, uint32_t threads,
                         hipStream_t s)
{
    hipError_t e;
    switch (p.node) {
    case 2: e = launch_partial<T, 2, NT>(p, grid1, threads, s); break;
    case 4: e = launch_partial<T, 4, NT>(p, grid1, threads, s); break;
    case 8: e = launch_partial<T, 8, NT>(p, grid1, threads, s); break;
    case 16: e = launch_partial<T, 16, NT>(p, grid1, threads, s); break;
    default: e = launch_partial<T, 0, NT>(p, grid1, threads, s); break;
    }
    if (e != hipSuccess)
        return e;
    switch (p.nodes) {
    case 2: return launch_fold<T, 2, NT>(p, grid2, threads, s);
    case 4: return launch_fold<T, 4, NT>(p, grid2, threads, s);
    case 8: return launch_fold<T, 8, NT>(p, grid2, threads, s);
    case 16: return launch_fold<T, 16, NT>(p, grid2, threads, s);
    default: return launch_fold<T, 0, NT>(p, grid2, threads, s);
    }
}

template <typename T>
hipError_t launch_dtype(const void *const *send, void *const *recv, size_t count, int nranks,
                        int group, void *ws, const HBConfig &cfg, int want_threads,
                        uint64_t want_blocks, bool nt, hipStream_t stream)
{
    constexpr uint64_t kPerVec = per_vec<T>();
    HierParams p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    p.ws = (float *)ws;
    p.pstride = hier_partial_stride(count) / 4;
    p.nvec = count / kPerVec;
    p.tail_elems = (uint32_t)(count % kPerVec);
    p.nranks = (uint32_t)nranks;
    p.node = (uint32_t)group;
    p.nodes = (uint32_t)(nranks / group);

    // Defaults: one-wave workgroups, four per CU, never more workgroups than
    // work items.  Measured at 16 and 32 ranks (fp32, 112 MiB per rank) and
    // 16 ranks (fp16, 8 MiB), this shape is the fastest of 64..512 threads x
    // 1..16 workgroups per CU for both stages together (3..15% under 256 x 1).
    uint32_t threads = want_threads > 0 ? (uint32_t)want_threads : 64u;
    if (threads > (uint32_t)kHierMaxThreads)
        threads = kHierMaxThreads;
    const uint64_t blocks = want_blocks > 0 ? want_blocks : 4 * (uint64_t)cfg.cu_count;
    const uint64_t tiles = (p.nvec + threads - 1) / threads;
    uint64_t grid1 = blocks < tiles * p.nodes ? blocks : tiles * p.nodes;
    uint64_t grid2 = blocks < tiles ? blocks : tiles;
    grid1 = grid1 < 1 ? 1 : grid1;
    grid2 = grid2 < 1 ? 1 : grid2;
    if (cfg.rec != nullptr)
        *cfg.rec = {arProtoHB, 2, (uint32_t)grid1, threads, 0, nt ? 1 : 0, group, 1};
    return nt ? launch_stages<T, true>(p, (uint32_t)grid1, (uint32_t)grid2, threads, stream)
              : launch_stages<T, false>(p, (uint32_t)grid1, (uint32_t)grid2, threads, stream);
}

}  // namespace

hipError_t launch_hb_hier(const void *const *send, void *const *recv, size_t count, int dtype,
                          int nranks, int group, void *ws, const HBConfig &cfg, int threads,
                          uint64_t blocks, bool nt, hipStream_t stream)
{
    switch (dtype) {
    case kBf16:
        return launch_dtype<Bf16>(send, recv, count, nranks, group, ws, cfg, threads, blocks, nt,
                                  stream);
    case kFp16:
        return launch_dtype<Fp16>(send, recv, count, nranks, group, ws, cfg, threads, blocks, nt,
                                  stream);
    default:
        return launch_dtype<Fp32>(send, recv, count, nranks, group, ws, cfg, threads, blocks, nt,
                                  stream);
    }
}

}  // namespace ar
