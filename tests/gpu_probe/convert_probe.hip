// convert_probe.hip -- test-only: the all-reduce kernels' fp32 -> bf16/fp16
// narrowing (ar::Bf16::narrow, ar::Fp16::narrow), applied to every binary32
// pattern in [start, start + n), so a GPU test can compare it with an
// independent converter.  Built with the library's own flags; not part of the
// library.
#include "ar_device.hpp"

__global__ __launch_bounds__(256) void narrow_patterns(int dtype, uint32_t start, uint64_t n,
                                                       uint16_t *out)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    float f[2] = {__builtin_bit_cast(float, (uint32_t)(start + (uint32_t)i)), 0.0f};
    const uint32_t w = dtype == 0 ? ar::Bf16::narrow(f) : ar::Fp16::narrow(f);
    out[i] = (uint16_t)w;
}

extern "C" int probe_narrow(int dtype, uint32_t start, uint64_t n, uint16_t *out, void *stream)
{
    if (n == 0 || (dtype != 0 && dtype != 1) || out == nullptr)
        return -1;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(narrow_patterns, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, dtype, start, n, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
