// qualify.hip -- test-only kernels that run the cast library's per-element
// device routines (csrc/device_math.h) over whole input domains, so that the
// GPU tests can compare every result with the oracle's rounding rules.  Not
// part of the library; built into tests/qualify/libqualify.so.
//
// Inputs are generated from the thread index (input i of a launch is the
// fp32 bit pattern first + i), so no input buffer is needed.  Pair routines
// (two inputs per instruction) are run with inputs i and i ^ 1 in both
// operand positions: pass `swap` = 0 puts the even input first, 1 the odd
// one; the per-input outputs of both passes must agree with the rule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"

using namespace mxk;

namespace {

__device__ __forceinline__ float in_bits(uint64_t v) { return __uint_as_float((uint32_t)v); }

// out[i] = the bf16 rounding of input i (uint16), for `pairs` input pairs.
__global__ void bf16_kernel(uint32_t first, int64_t pairs, int swap, uint16_t *out)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= pairs)
        return;
    const float x0 = in_bits((uint64_t)first + 2 * j), x1 = in_bits((uint64_t)first + 2 * j + 1);
    uint32_t w;
    if (swap) {
        w = bf16x2_rne(x1, x0);
        w = (w >> 16) | (w << 16);
    } else {
        w = bf16x2_rne(x0, x1);
    }
    reinterpret_cast<uint32_t *>(out)[j] = w;
}

// out[j] = the byte holding the E2M1 codes of inputs 2j (low nibble) and
// 2j + 1 (high nibble), taken from byte position j % 4 of the converted word.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_sel(float a, float b)
{
    return (e2m1x2<SEL>(a, b, 0u) >> (8 * SEL)) & 0xFFu;
}

__global__ void e2m1_kernel(uint32_t first, int64_t pairs, int swap, uint8_t *out)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= pairs)
        return;
    const float x0 = in_bits((uint64_t)first + 2 * j), x1 = in_bits((uint64_t)first + 2 * j + 1);
    const float a = swap ? x1 : x0, b = swap ? x0 : x1;
    uint32_t byte;
    switch (j & 3) {
    case 0: byte = e2m1_sel<0>(a, b); break;
    case 1: byte = e2m1_sel<1>(a, b); break;
    case 2: byte = e2m1_sel<2>(a, b); break;
    default: byte = e2m1_sel<3>(a, b); break;
    }
    if (swap)
        byte = (byte >> 4) | ((byte & 0xFu) << 4);
    out[j] = (uint8_t)byte;
}

// out[i] = the saturating E4M3 code of input i (e4m3x2: clamp to +-448 and
// the hardware convert), from the low (even j) or high (odd j) half.
__global__ void e4m3_kernel(uint32_t first, int64_t pairs, int swap, uint16_t *out)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= pairs)
        return;
    const float x0 = in_bits((uint64_t)first + 2 * j), x1 = in_bits((uint64_t)first + 2 * j + 1);
    const float a = swap ? x1 : x0, b = swap ? x0 : x1;
    uint32_t h = (j & 1) ? (e4m3x2<true>(a, b, 0u) >> 16) : (e4m3x2<false>(a, b, 0u) & 0xFFFFu);
    if (swap)
        h = (h >> 8) | ((h & 0xFFu) << 8);
    out[j] = (uint16_t)h;
}

// out[i] = exp32_nonpos(input i), bit pattern.
__global__ void exp_kernel(uint32_t first, int64_t n, uint32_t *out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    out[i] = __float_as_uint(exp32_nonpos(in_bits((uint64_t)first + i)));
}

// out[i] = rcp_1_2(d) for d = 1 + i * 2^-23, i = 0 .. 2^23 (every float in [1, 2]).
__global__ void rcp_kernel(uint32_t *out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i > (int64_t(1) << 23))
        return;
    out[i] = __float_as_uint(rcp_1_2(__uint_as_float(0x3F800000u + (uint32_t)i)));
}

// out[i] = div6_bf16(b) for the bf16 pattern i, i = 0 .. 0x7F7F (every finite
// non-negative bf16).
__global__ void div6_kernel(uint32_t *out)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i > 0x7F7F)
        return;
    out[i] = __float_as_uint(div6_bf16(__uint_as_float((uint32_t)i << 16)));
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

bool range_ok(uint32_t first, int64_t n)
{
    return n > 0 && n % 2 == 0 && (uint64_t)first + (uint64_t)n <= (uint64_t(1) << 32) &&
           (first & 1u) == 0;
}

}  // namespace

extern "C" {

// Each returns 0 on success, 1 for a bad range or NULL output, 2 for a launch
// error.  n inputs starting at pattern `first` (even, n even, first + n <=
// 2^32); outputs are device buffers of n elements (e2m1: n / 2 bytes).
int qual_bf16_rne(uint32_t first, int64_t n, int swap, uint16_t *out, hipStream_t s)
{
    if (!out || !range_ok(first, n))
        return 1;
    hipLaunchKernelGGL(bf16_kernel, dim3(blocks_for(n / 2)), dim3(256), 0, s, first, n / 2, swap,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int qual_e2m1(uint32_t first, int64_t n, int swap, uint8_t *out, hipStream_t s)
{
    if (!out || !range_ok(first, n))
        return 1;
    hipLaunchKernelGGL(e2m1_kernel, dim3(blocks_for(n / 2)), dim3(256), 0, s, first, n / 2, swap,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int qual_e4m3(uint32_t first, int64_t n, int swap, uint8_t *out, hipStream_t s)
{
    if (!out || !range_ok(first, n))
        return 1;
    hipLaunchKernelGGL(e4m3_kernel, dim3(blocks_for(n / 2)), dim3(256), 0, s, first, n / 2, swap,
                       reinterpret_cast<uint16_t *>(out));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int qual_exp(uint32_t first, int64_t n, uint32_t *out, hipStream_t s)
{
    if (!out || !range_ok(first, n))
        return 1;
    hipLaunchKernelGGL(exp_kernel, dim3(blocks_for(n)), dim3(256), 0, s, first, n, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out: (2^23 + 1) words.
int qual_rcp_1_2(uint32_t *out, hipStream_t s)
{
    if (!out)
        return 1;
    hipLaunchKernelGGL(rcp_kernel, dim3(blocks_for((int64_t(1) << 23) + 1)), dim3(256), 0, s, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out: 0x7F80 words.
int qual_div6(uint32_t *out, hipStream_t s)
{
    if (!out)
        return 1;
    hipLaunchKernelGGL(div6_kernel, dim3(blocks_for(0x7F80)), dim3(256), 0, s, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
