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

// div_by (division by a tensor-wide divisor) against the IEEE division.
// Thread i takes the divisor s = fp32 pattern first + i and every dividend
// the NVFP4 scale chain can give it: q = div6_bf16(b) for b = 0 and for every
// finite bf16 b whose quotient q / s lies in about [2^-12, 2^12].  Counts
// (summed over the launch): [0] quotients that differ from the IEEE q / s
// where that is at least 2^-10, [1] pairs whose E4M3 scale codes differ,
// [2] pairs tested.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

__global__ void divby_kernel(uint32_t first, int64_t n, unsigned long long *counts)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t bad_q = 0, bad_code = 0, tested = 0;
    if (i < n) {
        const float s = in_bits((uint64_t)first + i);
        const DivBy d = div_by_prepare(s);
        // b = 6 q spans [6 s 2^-12, 6 s 2^12]; positive bf16 patterns are
        // ordered like their values (an overflowing bound clamps to the
        // largest finite pattern)
        const uint32_t lo = __float_as_uint(6.0f * s * 0x1p-12f) >> 16;
        uint32_t hi = (__float_as_uint(6.0f * s * 0x1p12f) >> 16) + 1u;
        hi = hi > 0x7F7Fu ? 0x7F7Fu : hi;
        for (uint32_t p = lo == 0u ? 0u : lo - 1u; p <= hi; p++) {
            const uint32_t bp = p < lo ? 0u : p;   // the first pass takes b = 0
            const float q = div6_bf16(__uint_as_float(bp << 16));
            const float fast = div_by(q, d), ieee = q / s;
            bad_q += (__float_as_uint(fast) != __float_as_uint(ieee) && ieee >= 0x1p-10f) ? 1u : 0u;
            bad_code += ((e4m3x2<false>(fast, 0.0f, 0u) & 0xFFu) !=
                         (e4m3x2<false>(ieee, 0.0f, 0u) & 0xFFu)) ? 1u : 0u;
            tested++;
        }
    }
    bad_q = wave_sum(bad_q);
    bad_code = wave_sum(bad_code);
    tested = wave_sum(tested);
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&counts[0], (unsigned long long)bad_q);
        atomicAdd(&counts[1], (unsigned long long)bad_code);
        atomicAdd(&counts[2], (unsigned long long)tested);
    }
}

// out[i] = div_by(q[i], div_by_prepare(s[i])), for a CPU comparison.
__global__ void divby_values_kernel(const float *s, const float *q, int64_t n, float *out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    out[i] = div_by(q[i], div_by_prepare(s[i]));
}

// One wave multiplies two block-scaled operands the way a GEMM on gfx950
// consumes the cast's outputs: C[32][32] = sum over k of A[i][k] * B[k][j] by
// K / 64 steps of v_mfma_scale_f32_32x32x64_f8f6f4.
//   qa [32][K]: row-wise elements of a [32][K] tensor (A, blocks along k)
//   qb [32][K]: column-wise elements of a [K][32] tensor, i.e. B transposed
//               (row j holds B[.][j], blocks along k)
//   sa, sb:     their scales in the GEMM-ready tile layout (32 rows, so one
//               row tile; block tile bt at byte 256 bt)
// The instruction's operand layout (8-bit formats): lane L, h = L / 32,
// holds row L % 32, K values 16 h .. 16 h + 15 of each 32-value half of the
// step's 64 (bytes 0-15: k = 16 h + b; bytes 16-31: k = 32 + 16 h + b - 16);
// its scale byte scales K block h (k = 32 h .. 32 h + 31) of row L % 32.
// So lane L's scale word is word L of block tile t / 4, and byte t % 4 of it
// (the op_sel byte select) is the scale of step t.  FMT: 0 E4M3, 1 E5M2.
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

template <int FMT, int J>
__device__ __forceinline__ v16f_t mx_step(v8i_t a, v8i_t b, v16f_t c, int wa, int wb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, J, wa, J, wb);
}

template <int FMT>
__global__ void mfma_consumer_kernel(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb,
                                     const uint8_t *sb, int K, float *C)
{
    const int L = (int)threadIdx.x;        // one wave of 64
    v16f_t c = {};
    for (int t = 0; t < K / 64; t++) {
        const int k0 = 64 * t + 16 * (L >> 5);
        const uint4 a0 = *reinterpret_cast<const uint4 *>(qa + (L & 31) * K + k0);
        const uint4 a1 = *reinterpret_cast<const uint4 *>(qa + (L & 31) * K + k0 + 32);
        const uint4 b0 = *reinterpret_cast<const uint4 *>(qb + (L & 31) * K + k0);
        const uint4 b1 = *reinterpret_cast<const uint4 *>(qb + (L & 31) * K + k0 + 32);
        const v8i_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                         (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        const v8i_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                         (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const int wa = *reinterpret_cast<const int *>(sa + (t >> 2) * 256 + 4 * L);
        const int wb = *reinterpret_cast<const int *>(sb + (t >> 2) * 256 + 4 * L);
        switch (t & 3) {
        case 0: c = mx_step<FMT, 0>(a, b, c, wa, wb); break;
        case 1: c = mx_step<FMT, 1>(a, b, c, wa, wb); break;
        case 2: c = mx_step<FMT, 2>(a, b, c, wa, wb); break;
        default: c = mx_step<FMT, 3>(a, b, c, wa, wb); break;
        }
    }
    // accumulator layout of the 32 x 32 MFMA: lane L, register r holds
    // C[8 (r / 4) + 4 (L / 32) + r % 4][L % 32]
#pragma unroll
    for (int r = 0; r < 16; r++)
        C[(8 * (r >> 2) + 4 * (L >> 5) + (r & 3)) * 32 + (L & 31)] = c[r];
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

// Divisors first .. first + n - 1 (patterns of positive finite floats);
// counts: device, 3 zeroed uint64.
int qual_divby(uint32_t first, int64_t n, unsigned long long *counts, hipStream_t s)
{
    if (!counts || n <= 0 || (uint64_t)first + (uint64_t)n > 0x7F800000ull || first == 0u)
        return 1;
    hipLaunchKernelGGL(divby_kernel, dim3(blocks_for(n)), dim3(256), 0, s, first, n, counts);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// s, q, out: device arrays of n floats (s > 0 finite).
int qual_divby_values(const float *sv, const float *q, int64_t n, float *out, hipStream_t s)
{
    if (!sv || !q || !out || n <= 0)
        return 1;
    hipLaunchKernelGGL(divby_values_kernel, dim3(blocks_for(n)), dim3(256), 0, s, sv, q, n, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// qa, qb: device [32][K] element bytes; sa, sb: device tile-layout scales of
// 256 * K / 256 bytes each; K a positive multiple of 256; C: device [32][32]
// fp32.  fmt: 0 E4M3, 1 E5M2.  One wave.
int qual_mfma_consumer(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb,
                       const uint8_t *sb, int K, int fmt, float *C, hipStream_t s)
{
    if (!qa || !sa || !qb || !sb || !C || K <= 0 || K % 256 != 0 || (fmt != 0 && fmt != 1))
        return 1;
    if (fmt == 0)
        hipLaunchKernelGGL(mfma_consumer_kernel<0>, dim3(1), dim3(64), 0, s, qa, sa, qb, sb, K, C);
    else
        hipLaunchKernelGGL(mfma_consumer_kernel<1>, dim3(1), dim3(64), 0, s, qa, sa, qb, sb, K, C);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
