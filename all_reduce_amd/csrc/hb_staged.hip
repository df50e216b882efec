// hb_staged.hip -- the HB two-shot with its two shots as separate stages.
//
// The fused kernel (hb_twoshot.hip) needs no synchronisation at all on one
// GPU: the reduced vector goes from registers straight to all R outputs.
// Across R real GPUs the two shots of a reduce-scatter + all-gather
// ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南", blog.gitcode.com,
// section 4.4, rsag) are separated by a synchronisation: GPU c reduces chunk
// c into its own buffer, signals, and the peers then fetch the reduced chunk
// -- the HB protocol's rare synchronisation ("MSCCL++：让 GPU 通信像 CUDA 一样可编程",
// infinitensor.com/news/50, "MemoryChannel").  This file runs that staged
// form on one GPU, to measure what the stage boundary costs:
//   stage 1  for every position of chunk c: load the R inputs, reduce in
//            binary32 in rank order, store the result to rank c's output only;
//   (the kernel boundary is the signal)
//   stage 2  for every position of chunk c: load rank c's reduced value once
//            and store it to the other R - 1 outputs.
// Same result bits as the fused kernel; 2 * bytes-per-rank more HBM traffic
// (rank c's chunk is written, then read back) and one more launch.
//
// Chunks are interleaved tiles, as in the fused kernel's default layout:
// tile t (blockDim.x 16-byte vectors) belongs to chunk t % R.  In place is
// safe: in stage 1 only tile t's own workgroup reads tile t of any input, and
// stage 2 starts after stage 1 has finished.
#include "ar_device.hpp"
#include "ar_internal.hpp"

namespace ar {

template <int R>
struct StagedParams {
    RankTable<R> rk;
    uint64_t nvec;        // whole 16-byte vectors per rank
    uint32_t nranks;      // runtime rank count (the generic kernel; else == R)
    uint32_t tail_elems;  // elements after the last whole vector
};

constexpr int staged_max_threads(int rmax) { return rmax >= 32 ? 256 : (rmax >= 16 ? 512 : 1024); }

// The generic 32-slot table (17 to 31 ranks) is read from a wave-held copy
// (WaveTable), the run-time rank count re-read each tile, as in
// hb_twoshot_wave: in scalar registers its pointers and per-rank tests spill
// (48-74 lane writes per kernel).  The exact 32-rank kernels do not spill.
constexpr bool staged_wave_table(int rmax, bool exact) { return rmax >= 32 && !exact; }

template <typename T, int RMAX, bool EXACT, bool NT>
__global__ __launch_bounds__(staged_max_threads(RMAX)) void hb_stage_reduce(StagedParams<RMAX> p)
{
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint64_t tile = blockDim.x;
    const uint64_t ntiles = (p.nvec + tile - 1) / tile;
    constexpr bool kWT = staged_wave_table(RMAX, EXACT);
    WaveTable<RMAX> wt;
    if constexpr (kWT)
        wt = WaveTable<RMAX>(p.rk);
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        uint32_t nl = n;
        if constexpr (kWT) {
            wt.refresh();
            if constexpr (!EXACT)
                asm volatile("" : "+s"(nl));
        }
        const uint32_t c = (uint32_t)(t % nl);
        const uint64_t i = t * tile + threadIdx.x;
        if (i >= p.nvec)
            continue;
        u32x4 v[RMAX];
#pragma unroll
        for (int j = 0; j < RMAX; ++j)
            if (EXACT || j < (int)nl)
                v[j] = load16<NT>((const u32x4 *)(kWT ? wt.send(j) : p.rk.send[j]) + i);
        u32x4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float acc[T::kPerWord];
            T::widen(v[0][q], acc);
#pragma unroll
            for (int j = 1; j < RMAX; ++j) {
                if (EXACT || j < (int)nl) {
                    float x[T::kPerWord];
                    T::widen(v[j][q], x);
#pragma unroll
                    for (int e = 0; e < T::kPerWord; ++e)
                        acc[e] = acc[e] + x[e];
                }
            }
            y[q] = T::narrow(acc);
        }
        store16<NT>((u32x4 *)(kWT ? wt.recv(c) : p.rk.recv[c]) + i, y);
    }

    // Elements after the last whole vector: too few to stage; the last
    // workgroup writes them to every output here.
    if (p.tail_elems != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < p.tail_elems) {
        const uint64_t i = p.nvec * (16 / T::kBytes) + threadIdx.x;
        float a = 0.0f;
        uint32_t out = 0;
        for (uint32_t j = 0; j < n; ++j) {
            const uint32_t w = T::kBytes == 2 ? (uint32_t)((const uint16_t *)p.rk.send[j])[i]
                                              : ((const uint32_t *)p.rk.send[j])[i];
            float f[T::kPerWord];
            T::widen(w, f);
            a = j == 0 ? f[0] : a + f[0];
        }
        float f[T::kPerWord] = {};
        f[0] = a;
        out = T::narrow(f);
        for (uint32_t r = 0; r < n; ++r) {
            if (T::kBytes == 2)
                ((uint16_t *)p.rk.recv[r])[i] = (uint16_t)out;
            else
                ((uint32_t *)p.rk.recv[r])[i] = out;
        }
    }
}

template <int RMAX, bool EXACT, bool NT>
__global__ __launch_bounds__(staged_max_threads(RMAX)) void hb_stage_gather(StagedParams<RMAX> p)
{
    const uint32_t n = EXACT ? RMAX : p.nranks;
    const uint64_t tile = blockDim.x;
    const uint64_t ntiles = (p.nvec + tile - 1) / tile;
    constexpr bool kWT = staged_wave_table(RMAX, EXACT);
    WaveTable<RMAX> wt;
    if constexpr (kWT)
        wt = WaveTable<RMAX>(p.rk);
    for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        uint32_t nl = n;
        if constexpr (kWT) {
            wt.refresh();
            if constexpr (!EXACT)
                asm volatile("" : "+s"(nl));
        }
        const uint32_t c = (uint32_t)(t % nl);
        const uint64_t i = t * tile + threadIdx.x;
        if (i >= p.nvec)
            continue;
        const u32x4 y = load16<NT>((const u32x4 *)(kWT ? wt.recv(c) : p.rk.recv[c]) + i);
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
            if ((EXACT || r < (int)nl) && r != (int)c)
                store16<NT>((u32x4 *)(kWT ? wt.recv(r) : p.rk.recv[r]) + i, y);
    }
}

namespace {

template <typename T, int RMAX, bool EXACT, bool NT>
hipError_t launch_stages(const StagedParams<RMAX> &p, uint32_t grid, uint32_t threads,
                         hipStream_t stream)
{
    hipLaunchKernelGGL((hb_stage_reduce<T, RMAX, EXACT, NT>), dim3(grid), dim3(threads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nvec == 0)
        return e;
    hipLaunchKernelGGL((hb_stage_gather<RMAX, EXACT, NT>), dim3(grid), dim3(threads), 0, stream,
                       p);
    return hipGetLastError();
}

template <typename T, int RMAX, bool EXACT>
hipError_t launch_table(const void *const *send, void *const *recv, size_t count, int nranks,
                        const HBConfig &cfg, int want_threads, uint64_t want_blocks, bool nt,
                        hipStream_t stream)
{
    constexpr uint64_t kPerVec = 16 / T::kBytes;
    StagedParams<RMAX> p = {};
    for (int r = 0; r < nranks; ++r) {
        p.rk.send[r] = send[r];
        p.rk.recv[r] = recv[r];
    }
    p.nvec = count / kPerVec;
    p.tail_elems = (uint32_t)(count % kPerVec);
    p.nranks = (uint32_t)nranks;
    // The fused kernel's defaults: 256 threads (128 from 32 ranks up), one
    // workgroup per CU, but never more workgroups than tiles.
    uint32_t threads = want_threads > 0 ? (uint32_t)want_threads : (nranks >= 32 ? 128u : 256u);
    if (threads > (uint32_t)staged_max_threads(RMAX))
        threads = (uint32_t)staged_max_threads(RMAX);
    uint64_t grid = want_blocks > 0 ? want_blocks : (uint64_t)cfg.cu_count;
    const uint64_t ntiles = (p.nvec + threads - 1) / threads;
    if (grid > ntiles)
        grid = ntiles;
    if (grid < 1)
        grid = 1;
    if (cfg.rec != nullptr)
        *cfg.rec = {arProtoHB, p.nvec == 0 ? 1 : 2, (uint32_t)grid, threads, 0, nt ? 1 : 0, 0, 1};
    return nt ? launch_stages<T, RMAX, EXACT, true>(p, (uint32_t)grid, threads, stream)
              : launch_stages<T, RMAX, EXACT, false>(p, (uint32_t)grid, threads, stream);
}

template <typename T>
hipError_t launch_dtype(const void *const *send, void *const *recv, size_t count, int nranks,
                        const HBConfig &cfg, int th, uint64_t bl, bool nt, hipStream_t stream)
{
    switch (nranks) {
    case 1: return launch_table<T, 1, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    case 2: return launch_table<T, 2, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    case 4: return launch_table<T, 4, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    case 8: return launch_table<T, 8, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    case 16: return launch_table<T, 16, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    case 32: return launch_table<T, 32, true>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    default: break;
    }
    if (nranks < 8)
        return launch_table<T, 8, false>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    if (nranks < 16)
        return launch_table<T, 16, false>(send, recv, count, nranks, cfg, th, bl, nt, stream);
    return launch_table<T, 32, false>(send, recv, count, nranks, cfg, th, bl, nt, stream);
}

}  // namespace

hipError_t launch_hb_staged(const void *const *send, void *const *recv, size_t count, int dtype,
                            int nranks, const HBConfig &cfg, int threads, uint64_t blocks, bool nt,
                            hipStream_t stream)
{
    switch (dtype) {
    case kBf16:
        return launch_dtype<Bf16>(send, recv, count, nranks, cfg, threads, blocks, nt, stream);
    case kFp16:
        return launch_dtype<Fp16>(send, recv, count, nranks, cfg, threads, blocks, nt, stream);
    default:
        return launch_dtype<Fp32>(send, recv, count, nranks, cfg, threads, blocks, nt, stream);
    }
}

}  // namespace ar
