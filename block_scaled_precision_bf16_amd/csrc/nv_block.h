// nv_block.h -- the arithmetic of one NVFP4 block, shared by the NVFP4
// kernels (nvfp4.hip: the tiled quantize-transpose, nvfp4_any.hip: any
// shape): the tensor's global scale, a block's E4M3 scale byte, the
// element multiplier of a scale byte, and the E2M1 codes of eight elements.
#pragma once

#include "device_math.h"

namespace mxk {

// The global scale of a tensor with amax A: A / (448 * 6), 1 for A = 0.
__device__ __forceinline__ float nv_global_scale(float A) { return A == 0.0f ? 1.0f : A / 2688.0f; }

// Scale byte of one NVFP4 block whose largest magnitude has bf16 pattern
// mag: E4M3(fl32(fl32(b / 6) / S_g)).  The division by S_g gives the IEEE
// quotient wherever the code can be non-zero (div_by, prepared once per
// workgroup); the E4M3 rounding is the saturating hardware convert (inputs
// are finite here).
__device__ __forceinline__ uint32_t nv_scale(uint32_t mag, const DivBy &sg)
{
    const float sq = div_by(div6_bf16(f32_bits(mag << 16)), sg);
    return e4m3x2<false>(sq, 0.0f, 0u) & 0xFFu;
}

// Element multiplier of scale byte s: fl32(1 / fl32(dec(s) * S_g)), 0 when
// the product is 0.  It depends on s alone within a tensor, so a workgroup
// tabulates the 127 finite codes once.
__device__ __forceinline__ float nv_inverse(uint32_t s, float sg)
{
    const float den = e4m3_value(s) * sg;
    return den == 0.0f ? 0.0f : 1.0f / den;
}

// 0xF when bf16 h is +-0 or NaN (its product with an infinite multiplier is
// NaN), else 0.
__device__ __forceinline__ uint32_t zero_or_nan_nibble(uint32_t h)
{
    const uint32_t a = h & 0x7FFFu;
    return (a == 0u || a > 0x7F80u) ? 0xFu : 0u;
}

// Eight bf16 (four words) times inv -> eight E2M1 nibbles, element i in bits
// 4i..4i+3 (so element 2j is the low nibble of byte j).  The hardware
// convert gives the nearest E2M1 code on every non-NaN product (e2m1x2); a
// NaN product (0 * Inf or NaN * Inf, possible only when the multiplier
// overflowed to Inf, tensor scale below ~2^-120) must encode as +0, so such
// nibbles are cleared afterwards.
__device__ __forceinline__ uint32_t encode8_fp4(const uint32_t (&w)[4], float inv)
{
    uint32_t o = e2m1x2<0>(bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, 0u);
    o = e2m1x2<1>(bf16_lo(w[1]) * inv, bf16_hi(w[1]) * inv, o);
    o = e2m1x2<2>(bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, o);
    o = e2m1x2<3>(bf16_lo(w[3]) * inv, bf16_hi(w[3]) * inv, o);
    const bool inf = __builtin_isinf(inv);
    if (__builtin_amdgcn_ballot_w64(inf) != 0) {   // uniform: no lane's exec mask changes
        uint32_t clear = 0;
#pragma unroll
        for (int d = 0; d < 4; d++)
            clear |= (zero_or_nan_nibble(w[d]) << (8 * d)) | (zero_or_nan_nibble(w[d] >> 16) << (8 * d + 4));
        o &= inf ? ~clear : ~0u;
    }
    return o;
}

}  // namespace mxk
