/*
 * oracle.c -- plain CPU reference for the sum all-reduce over R rank buffers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the tests, the smoke check of the entry module and the
 * CPU-baseline leg of the benchmark use it.  It shares no source, header,
 * table or helper with the HIP library under all_reduce_amd/csrc.
 *
 * What it computes (one definition, no blocking, fusion or reordering):
 *
 *   for every element index i in [0, count):
 *       a    = widen(x_0[i])                    exact (bf16/fp16 -> fp32)
 *       a    = fl32(a + widen(x_j[i]))   for j = 1 .. R-1, in that order,
 *                                       each an IEEE-754 binary32 add, RNE
 *       y[i] = narrow_rne(a)                    fp32 -> bf16/fp16, RNE;
 *                                               identity for fp32
 *       out_r[i] = y[i]                  for every rank r = 0 .. R-1
 *
 * Sources:
 *  - SUM is the only reduction and float/float16/bfloat16 the only dtypes:
 *    "SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南" (blog.gitcode.com),
 *    section 4.3 (runtime guard conditions 2 and 4) and section 5.
 *  - Every rank ends with the same summed vector (an all-reduce replaces
 *    ncclAllReduce one for one): "MSCCL++：让 GPU 通信像 CUDA 一样可编程"
 *    (infinitensor.com/news/50), section "第一层：Collective API"; the LL and HB
 *    protocols of its "MemoryChannel" table are two ways to the same result.
 *  - The pages fix neither the summation order, nor the accumulator type, nor
 *    the rounding.  The reading taken here: ranks summed in the fixed order
 *    0..R-1, accumulator starting from x_0 itself (so an all -0 column gives
 *    -0), binary32 accumulation, round-to-nearest-even narrowing.  With a
 *    fixed order the result is unique, so a kernel that keeps the order must
 *    match bit for bit.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * x86-64 float arithmetic is SSE binary32 with RNE; MXCSR FTZ/DAZ stay off,
 * so subnormals follow IEEE gradual underflow.  Each element is computed by
 * exactly one thread, so the output bits do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1, ORACLE_FP32 = 2 };

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bfloat16 is the upper half of a binary32 word: widening is a shift. */
float oracle_widen_bf16(uint16_t h)
{
    return f32_from_bits((uint32_t)h << 16);
}

/* binary16: value = (-1)^s * 2^(e-15) * (1 + m/1024) for 1 <= e <= 30,
 * (-1)^s * 2^-14 * (m/1024) for e = 0, inf/NaN for e = 31.  Every binary16
 * value is exactly representable in binary32, so ldexpf is exact here. */
float oracle_widen_fp16(uint16_t h)
{
    uint32_t s = (h >> 15) & 1u;
    uint32_t e = (h >> 10) & 0x1fu;
    uint32_t m = h & 0x3ffu;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -24);
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexpf((float)(m | 0x400u), (int)e - 25);
    return s ? -mag : mag;
}

/* fp32 -> bf16, round to nearest, ties to even, on the 16 dropped bits.
 * A carry out of the kept mantissa moves into the exponent, which is the
 * correct result (the largest finite values round up to infinity).  NaN keeps
 * its sign and upper payload bits and is forced quiet. */
uint16_t oracle_rne_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* fp32 -> binary16, round to nearest, ties to even, with gradual underflow.
 * The finite input is sig * 2^(E-23) with a 24-bit significand sig.  The
 * binary16 quantum at that magnitude is 2^Q with Q = max(E, -14) - 10; the
 * result is the nearest multiple of 2^Q (ties to an even multiple).  Counted
 * in quanta q, a normal result is ((E+15) << 10) + q - 1024 -- a round-up to
 * q = 2048 carries into the exponent, and past the largest exponent that
 * carry lands on the infinity encoding -- and a subnormal result is q. */
uint16_t oracle_rne_fp16(float f)
{
    uint32_t u = bits_from_f32(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t absu = u & 0x7fffffffu;
    if (absu > 0x7f800000u)                                  /* NaN */
        return (uint16_t)(sign | 0x7e00u | ((absu >> 13) & 0x1ffu));
    if (absu == 0x7f800000u)                                 /* infinity */
        return (uint16_t)(sign | 0x7c00u);
    if (absu == 0)
        return sign;

    int biased = (int)(absu >> 23);
    uint64_t sig = absu & 0x7fffffu;
    int E;
    if (biased == 0) {            /* binary32 subnormal: 0.m * 2^-126 */
        E = -126;
    } else {
        E = biased - 127;
        sig |= 0x800000u;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00u);                   /* overflow */

    int Q = (E > -14 ? E : -14) - 10;
    int shift = Q - (E - 23);                                /* >= 13 */
    uint64_t q;
    if (shift > 40) {
        q = 0;                                               /* < half quantum */
    } else {
        q = sig >> shift;
        uint64_t rem = sig & ((1ull << shift) - 1u);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (q & 1u)))
            q += 1u;
    }
    uint32_t bits;
    if (E < -14)
        bits = (uint32_t)q;
    else
        bits = ((uint32_t)(E + 15) << 10) + (uint32_t)q - 1024u;
    return (uint16_t)(sign | bits);
}

/* The sum all-reduce.  send[r] / recv[r] point at rank r's count elements.
 * recv[r] == send[r] (in place) is allowed: element i of every rank is read
 * before element i of any rank is written, and only one thread touches i.
 * Returns 0 on success, -1 on an unknown dtype or nranks < 1. */
int oracle_allreduce(const void *const *send, void *const *recv, size_t count,
                     int dtype, int nranks, int nthreads)
{
    if (nranks < 1 || dtype < ORACLE_BF16 || dtype > ORACLE_FP32)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    const ptrdiff_t n = (ptrdiff_t)count;

    if (dtype == ORACLE_BF16) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (ptrdiff_t i = 0; i < n; ++i) {
            float a = oracle_widen_bf16(((const uint16_t *)send[0])[i]);
            for (int j = 1; j < nranks; ++j)
                a = a + oracle_widen_bf16(((const uint16_t *)send[j])[i]);
            uint16_t y = oracle_rne_bf16(a);
            for (int r = 0; r < nranks; ++r)
                ((uint16_t *)recv[r])[i] = y;
        }
    } else if (dtype == ORACLE_FP16) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (ptrdiff_t i = 0; i < n; ++i) {
            float a = oracle_widen_fp16(((const uint16_t *)send[0])[i]);
            for (int j = 1; j < nranks; ++j)
                a = a + oracle_widen_fp16(((const uint16_t *)send[j])[i]);
            uint16_t y = oracle_rne_fp16(a);
            for (int r = 0; r < nranks; ++r)
                ((uint16_t *)recv[r])[i] = y;
        }
    } else {
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (ptrdiff_t i = 0; i < n; ++i) {
            float a = ((const float *)send[0])[i];
            for (int j = 1; j < nranks; ++j)
                a = a + ((const float *)send[j])[i];
            for (int r = 0; r < nranks; ++r)
                ((float *)recv[r])[i] = a;
        }
    }
    return 0;
}

/* Hierarchical (two-level) order: ranks form nranks / group consecutive
 * groups ("nodes") of `group` ranks.  For every element, each group's partial
 * sum is taken in binary32 in rank order within the group, starting from the
 * group's first rank; the partials are then summed in binary32 in group
 * order, starting from group 0's; the result is rounded once (RNE).  This is
 * the order of an all-reduce that reduces inside each node first and across
 * nodes second ("SGLang 中的 MSCCL++ All-Reduce 基准测试与推理集成指南",
 * blog.gitcode.com, section 4.4: multi-node algorithms for TP = 16 / 32),
 * with the cross-node partials kept in binary32.  group == nranks (and
 * group == 1) is the flat order of oracle_allreduce.
 * Returns 0, or -1 on an unknown dtype, nranks < 1, group < 1 or a group that
 * does not divide nranks. */
static float grouped_sum(const void *const *send, ptrdiff_t i, int dtype, int nranks, int group)
{
    float total = 0.0f;
    for (int g = 0; g < nranks / group; ++g) {
        float part = 0.0f;
        for (int l = 0; l < group; ++l) {
            const int j = g * group + l;
            float x;
            if (dtype == ORACLE_BF16)
                x = oracle_widen_bf16(((const uint16_t *)send[j])[i]);
            else if (dtype == ORACLE_FP16)
                x = oracle_widen_fp16(((const uint16_t *)send[j])[i]);
            else
                x = ((const float *)send[j])[i];
            part = (l == 0) ? x : part + x;
        }
        total = (g == 0) ? part : total + part;
    }
    return total;
}

int oracle_allreduce_grouped(const void *const *send, void *const *recv, size_t count,
                             int dtype, int nranks, int group, int nthreads)
{
    if (nranks < 1 || group < 1 || nranks % group != 0 || dtype < ORACLE_BF16 ||
        dtype > ORACLE_FP32)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (ptrdiff_t i = 0; i < (ptrdiff_t)count; ++i) {
        const float a = grouped_sum(send, i, dtype, nranks, group);
        for (int r = 0; r < nranks; ++r) {
            if (dtype == ORACLE_BF16)
                ((uint16_t *)recv[r])[i] = oracle_rne_bf16(a);
            else if (dtype == ORACLE_FP16)
                ((uint16_t *)recv[r])[i] = oracle_rne_fp16(a);
            else
                ((float *)recv[r])[i] = a;
        }
    }
    return 0;
}

/* Array forms of the converters, for the exhaustive converter pins. */
void oracle_rne_bf16_array(const float *in, uint16_t *out, size_t n, int nthreads)
{
#pragma omp parallel for num_threads(nthreads < 1 ? 1 : nthreads) schedule(static)
    for (ptrdiff_t i = 0; i < (ptrdiff_t)n; ++i)
        out[i] = oracle_rne_bf16(in[i]);
}

void oracle_rne_fp16_array(const float *in, uint16_t *out, size_t n, int nthreads)
{
#pragma omp parallel for num_threads(nthreads < 1 ? 1 : nthreads) schedule(static)
    for (ptrdiff_t i = 0; i < (ptrdiff_t)n; ++i)
        out[i] = oracle_rne_fp16(in[i]);
}

void oracle_widen_fp16_array(const uint16_t *in, float *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_widen_fp16(in[i]);
}

/* Wall time of one oracle_allreduce call, in seconds, measured with the
 * monotonic OpenMP clock around the call only (no input generation). */
double oracle_allreduce_timed(const void *const *send, void *const *recv,
                              size_t count, int dtype, int nranks, int nthreads)
{
    double t0 = omp_get_wtime();
    int rc = oracle_allreduce(send, recv, count, dtype, nranks, nthreads);
    double t1 = omp_get_wtime();
    return rc == 0 ? t1 - t0 : -1.0;
}
