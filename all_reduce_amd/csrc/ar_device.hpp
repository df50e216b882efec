// ar_device.hpp -- device-side building blocks shared by the LL and HB kernels.
//
// Element handling for the sum all-reduce of bfloat16, float16 and float32
// buffers (the dtypes admitted by the runtime guards of the SGLang MSCCL++
// all-reduce guide, blog.gitcode.com, section 4.3):
//
//  * data moves as 32-bit words (LL packet payloads) or 128-bit vectors (HB);
//  * the R simulated ranks' buffers reach a kernel as a table of pointers;
//  * each element is widened to binary32 exactly, summed in rank order
//    0..R-1 starting from rank 0's value, and narrowed once with round to
//    nearest even.
//
// Narrowing uses gfx950's packed converts (v_cvt_pk_bf16_f32,
// v_cvt_pk_f16_f32).  They round with the wave's float mode, which the kernel
// descriptor leaves at round-to-nearest-even with binary32 denormals kept
// (the library is built with -fno-gpu-flush-denormals-to-zero).  The GPU
// tests check them against an independent converter over all 2^32 inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per-dtype word handling.  kPerWord elements fill one 32-bit word; kId is
// the dtype's arDataType_t value.
struct Bf16 {
    static constexpr int kId = 0;
    static constexpr int kPerWord = 2;
    static constexpr int kBytes = 2;
    __device__ static inline void widen(uint32_t w, float *f)
    {
        f[0] = __builtin_bit_cast(float, w << 16);          // low element
        f[1] = __builtin_bit_cast(float, w & 0xffff0000u);  // high element
    }
    __device__ static inline uint32_t narrow(const float *f)
    {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
};

struct Fp16 {
    static constexpr int kId = 1;
    static constexpr int kPerWord = 2;
    static constexpr int kBytes = 2;
    __device__ static inline void widen(uint32_t w, float *f)
    {
        f32x2 v = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        f[0] = v.x;
        f[1] = v.y;
    }
    __device__ static inline uint32_t narrow(const float *f)
    {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
};

struct Fp32 {
    static constexpr int kId = 2;
    static constexpr int kPerWord = 1;
    static constexpr int kBytes = 4;
    __device__ static inline void widen(uint32_t w, float *f) { f[0] = __builtin_bit_cast(float, w); }
    __device__ static inline uint32_t narrow(const float *f) { return __builtin_bit_cast(uint32_t, f[0]); }
};

// 128-bit global loads and stores, optionally non-temporal (streamed data
// that is touched once should not displace other lines in L2 / MALL).
template <bool NT>
__device__ inline u32x4 load16(const u32x4 *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT>
__device__ inline void store16(u32x4 *p, u32x4 v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Rank pointer table, passed by value in the kernel arguments: the host-built
// "channels" of the simulated group (the microsoft/mscclpp project summary,
// agentlenshq.com, "How it works": channels are set up on the host and used
// from device code).  Sized for the kernel's compile-time rank count.
template <int R>
struct RankTable {
    const void *send[R];
    void *recv[R];
};

// The same table held by a wave, one entry per lane: lane r < R holds send[r],
// lane 32 + r holds recv[r].  A pointer is read back with two lane reads where
// it is used, so that the table never sits in scalar registers whole: 32
// ranks' 64 pointers need 128 of them, more than a wave has, and the compiler
// then spills and reloads them in blocks around every use.  The pointers come
// back through a global-memory pointer so that accesses stay global ones
// (a pointer rebuilt from integers would otherwise be a flat one).  Every wave
// must be whole (64 lanes): the kernels that use it are launched with
// workgroups of a multiple of 64 threads, which the options check enforces.
template <int R>
struct WaveTable {
    static_assert(R <= 32, "one wave holds at most 32 send and 32 recv pointers");
    uint64_t v = 0;
    WaveTable() = default;
    __device__ explicit WaveTable(const RankTable<R> &t)
    {
        const uint32_t lane = __lane_id();
        const uint32_t r = lane & 31u;
        uint64_t e = 0;
        if (r < (uint32_t)R)
            e = lane < 32u ? (uint64_t)t.send[r] : (uint64_t)t.recv[r];
        v = e;
        // The load completes here, not at the top of a loop that uses it,
        // where the wait would also take in the loop's own stores.
        asm volatile("" : "+v"(v));
    }
    // Called at the top of a loop: keeps the compiler from hoisting the lane
    // reads out of it, which would bring back the scalar-register table.
    __device__ void refresh() { asm volatile("" : "+v"(v)); }
    __device__ uint64_t get(int lane) const
    {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
        return ((uint64_t)hi << 32) | lo;
    }
    __device__ const void *send(int r) const
    {
        return (const void *)(const __attribute__((address_space(1))) char *)get(r);
    }
    __device__ void *recv(int r) const
    {
        return (void *)(__attribute__((address_space(1))) char *)get(32 + r);
    }
};

}  // namespace ar
