// device_math.h -- per-element and per-block arithmetic of the cast kernels
// (gfx950).  Everything here is exact integer work or a fixed sequence of
// IEEE fp32 operations, so results are reproducible bit for bit.  The whole
// library is compiled with -ffp-contract=off: every a*b+c below is two
// roundings unless written as __builtin_fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mxk {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f32_bits(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t bits_f32(float f) { return __float_as_uint(f); }

// bf16 halves of a packed word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return f32_bits(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return f32_bits(w & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> a packed pair of bf16 bits (lo in bits 0-15), round to nearest
// even, by gfx950's v_cvt_pk_bf16_f32: on every one of the 2^32 fp32 inputs,
// in either half of the pair, the nearest bf16 with ties to even (overflow to
// Inf; NaN stays NaN), as the device qualification tests check against the
// oracle's rounding.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    const bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Lane-wise max of the two 15-bit magnitudes packed in a word of bf16 pairs.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

// Exponent of the element format's largest binade (format flags: launch.h).
template <int FMT>
constexpr uint32_t fmt_emax() { return (FMT & kFmtE5M2) ? 15u : 8u; }

// ---------------------------------------------------------------------------
// MX scale: E8M0 byte from the largest |bf16| of a block, given as its
// 15-bit magnitude pattern.  For a finite amax the exponent field E equals
// floor(log2 amax) + 127 (normal) or 0 (subnormal, where the clamp applies).
//   floor rule:    byte = max(E - emax, 0)
//   round-up rule: byte = max(E - emax + (mantissa > 0x60), 0), since
//                  ceil(log2(amax / (1.75 * 2^emax))) = E - 127 - emax exactly
//                  when the 7-bit mantissa is at most 0x60 (1 + 96/128 = 1.75)
//                  and one more otherwise.
// Inf / NaN (pattern >= 0x7F80) -> 0xFF.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ uint32_t scale_byte(uint32_t mag)
{
    int e = (int)(mag >> 7) - (int)fmt_emax<FMT>();
    if constexpr ((FMT & kFmtRoundUp) != 0)
        e += (mag & 0x7Fu) > 0x60u ? 1 : 0;
    uint32_t b = e > 0 ? (uint32_t)e : 0u;
    return mag >= 0x7F80u ? 0xFFu : b;
}

// Two fp32 -> two E4M3 bytes (round to nearest even, saturating), written into
// the low (HI = false) or high (HI = true) 16 bits of `old`, first value in the
// lower byte.  v_cvt_pk_fp8_f32 rounds to nearest even but turns values beyond
// the format into NaN, so both inputs are first clamped to +-448, which leaves
// every in-range value (and -0) unchanged.  The device qualification tests
// compare the pair, in both halves and both operand positions, with the
// oracle's saturating E4M3 rounding on every non-NaN fp32 input.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2(float a, float b, uint32_t old)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Lane-wise min of two packed 16-bit magnitudes.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(va, vb));
}

// bf16 pattern of the largest magnitude a block with scale byte b may keep
// before saturating: max * 2^(b - 127) = 1.75 * 2^(b + emax - 127), i.e.
// exponent field b + emax and mantissa 0x60, duplicated into both halves.
// Valid for b <= 254 - emax, the largest byte the floor rule gives a finite
// bf16 amax.  (Under the round-up rule nothing exceeds the limit.)
template <int FMT = 0>
__device__ __forceinline__ uint32_t sat_limit2(uint32_t b)
{
    const uint32_t l = ((b + fmt_emax<FMT>()) << 7) | 0x60u;
    return l | (l << 16);
}

// A packed pair of bf16 with each magnitude clamped to the limit (signs kept).
__device__ __forceinline__ uint32_t clamp_pair(uint32_t w, uint32_t mag, uint32_t lim2)
{
    return (pk_min_u16(mag, lim2) & 0x7FFF7FFFu) | (w & 0x80008000u);
}

// A packed pair of bf16 -> two E4M3 bytes in the low (HI = false) or high
// 16 bits of `old`, first element in the lower byte.  The pair must already be
// clamped with sat_limit2(b); v_cvt_scalef32_pk_fp8_bf16 then divides each
// element by 2^(b - 127) -- the scale operand carries the E8M0 byte in its
// exponent field -- and rounds to nearest even, which is exactly the block
// rule (the division by a power of two is exact, so it equals multiplying by
// the inverse).  The clamp is what makes it saturate: on its own the
// instruction turns values beyond 448 into NaN.  The exhaustive parity tensor
// of the GPU tests (every finite bf16 element under every scale byte it can
// meet, in both halves of a pair) checks the result against the oracle's
// nearest-E4M3 rule bit for bit.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_scaled(uint32_t pair, float scale, uint32_t old)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2, old),
                                                              __builtin_bit_cast(bf16x2, pair),
                                                              scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// The same for E5M2 elements (v_cvt_scalef32_pk_bf8_bf16: round to nearest
// even, subnormals kept; the caller clamps to 57344 * 2^(b - 127) first under
// the floor rule).  Checked against the nearest-E5M2 rule over every reachable
// (element, byte) pair by the exhaustive parity tensors.
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_scaled(uint32_t pair, float scale, uint32_t old)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(__builtin_bit_cast(s16x2, old),
                                                              __builtin_bit_cast(bf16x2, pair),
                                                              scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// Element conversion of a packed bf16 pair (magnitudes mag) in the block
// format FMT with scale byte b (operand sc = e8m0_operand(b), limit lim =
// sat_limit2<FMT>(b)).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t mx_pair(uint32_t w, uint32_t mag, uint32_t lim, float sc,
                                            uint32_t old)
{
    const uint32_t p = (FMT & kFmtRoundUp) ? w : clamp_pair(w, mag, lim);
    if constexpr ((FMT & kFmtE5M2) != 0)
        return e5m2x2_scaled<HI>(p, sc, old);
    else
        return e4m3x2_scaled<HI>(p, sc, old);
}

// The scale operand of the scaled converts: the E8M0 byte in the exponent field.
__device__ __forceinline__ float e8m0_operand(uint32_t b) { return f32_bits(b << 23); }

// Two fp32 -> two E2M1 nibbles in byte SEL of `old` (first value in the low
// nibble), by v_cvt_scalef32_pk_fp4_f32 with scale 1: round to nearest even,
// saturating at 6, Inf -> 6.  The device qualification tests compare it, in
// all four byte positions and both operand positions, with the oracle's E2M1
// rounding on every non-NaN fp32 input.  (A NaN input -- only 0 * Inf -- is
// not covered; callers clear the nibbles of such products.)
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2(float a, float b, uint32_t old)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// fl32(b / 6) for b >= 0 holding a bf16 value (at most 8 significant bits):
// q0 = b * RN(1/6), the residual b - 6 q0 (exact in the FMA, since q0 is
// within an ulp of b / 6), and one correction step.  Equal to the IEEE
// division for every finite non-negative bf16 (shown with exact rational
// arithmetic by the CPU tests, and compared on the device with the correctly
// rounded quotient by the qualification tests), at a third of its cost.
__device__ __forceinline__ float div6_bf16(float b)
{
    const float c = 0x1.555556p-3f;   // RN(1/6)
    const float q0 = b * c;
    const float r = __builtin_fmaf(-6.0f, q0, b);
    return __builtin_fmaf(r, c, q0);
}

// Division by a divisor s > 0 that is fixed for a whole tensor, without the
// per-call IEEE sequence (two scale steps, a reciprocal estimate, five FMAs
// and a fix-up).  Prepared once: k = 2^64 for s < 2^-90, else 1; s' = s k
// (exact) and y = fl32(1 / s') by the IEEE division.  Per call, with q' = q k
// (exact): q0 = q' y, then twice q_i+1 = q_i + (q' - s' q_i) y, the residual
// exact in the FMA.  The final step from a quotient within an ulp and a
// correctly rounded reciprocal gives the correctly rounded quotient
// (Markstein's theorem) wherever the residuals stay normal: for every q whose
// quotient q / s is at least 2^-10 (the smallest value the E4M3 scale can
// take), since s' >= 2^-90 bounds the residuals from below.  The device
// qualification tests compare it with the IEEE quotient over every divisor
// mantissa at both ends of the range and every subnormal divisor.
struct DivBy {
    float s, y, k;
};

__device__ __forceinline__ DivBy div_by_prepare(float s)
{
    DivBy d;
    d.k = s < 0x1p-90f ? 0x1p64f : 1.0f;
    d.s = s * d.k;
    d.y = 1.0f / d.s;
    return d;
}

__device__ __forceinline__ float div_by(float q, const DivBy &d)
{
    const float qk = q * d.k;
    const float q0 = qk * d.y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-d.s, q0, qk), d.y, q0);
    return __builtin_fmaf(__builtin_fmaf(-d.s, q1, qk), d.y, q1);
}

// E4M3 code (no NaN) -> its exact fp32 value.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float mag = e ? f32_bits(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Fused pre-op arithmetic.  Each statement is one IEEE fp32 operation.
// ---------------------------------------------------------------------------

// e^a for a <= 0 (or NaN), the only arguments the activations need: Cody &
// Waite reduction a = n ln2 + r (ln2 = 355/512 + remainder), the degree-7
// Taylor polynomial of e^r by Horner with fused multiply-adds, and scaling by
// 2^n with one final rounding (also for subnormal results).  Arguments are
// clamped at -104, where the sequence already gives 0 (0.97 * 2^-150 rounds
// to 0), so every smaller argument gets that same 0 without a select; NaN
// propagates through the final select.  KEEP_NAN = false leaves that select
// out (a NaN argument then gives 0), for callers whose result is NaN anyway.
template <bool KEEP_NAN = true>
__device__ __forceinline__ float exp32_nonpos(float a)
{
    const float LOG2E = 1.44269504088896340736f;
    const float LN2_A = 0.693359375f;                 // 355/512
    const float LN2_B = -2.12194440054690583e-4f;     // ln2 - 355/512
    const float LO = -104.0f;
    const float c = __builtin_fmaxf(a, LO);
    const float n = __builtin_rintf(c * LOG2E);
    float r = __builtin_fmaf(n, -LN2_A, c);
    r = __builtin_fmaf(n, -LN2_B, r);
    float p = (float)(1.0 / 5040.0);
    p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
    p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    // p * 2^n with one rounding (v_ldexp_f32, denormals kept): the same bits
    // as scaling by 2^(n/2) and then 2^(n - n/2), the first product exact
    const float e = __builtin_amdgcn_ldexpf(p, (int)n);    // n in [-150, 0]
    if constexpr (KEEP_NAN)
        return a != a ? a : e;
    return e;
}

// fl32(1 / d) for d in [1, 2]: the hardware reciprocal estimate and one
// Newton step with FMAs, at a third of the cost of the IEEE division and equal
// to it for every one of the 2^23 + 1 floats in [1, 2] (the device
// qualification tests compare all of them with the correctly rounded
// quotient).
__device__ __forceinline__ float rcp_1_2(float d)
{
    const float r0 = __builtin_amdgcn_rcpf(d);
    return __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
}

// sigma(z) = 1/(1+e^-z) and 1 - sigma(z) from e = e^-|z| (no overflow, no
// cancellation): z >= 0 gives (1/(1+e), e/(1+e)), z < 0 the swapped pair.
__device__ __forceinline__ void sigmoid_pair(float z, float &s, float &sc)
{
    float e = exp32_nonpos(-__builtin_fabsf(z));
    float d = 1.0f + e;
    float r = rcp_1_2(d);   // d is in [1, 2]
    float er = e * r;
    s = z >= 0.0f ? r : er;
    sc = z >= 0.0f ? er : r;
}

// sigma(z) alone, for the forward activations x * sigma(.).  The exp's NaN
// select is left out: z is NaN only when x is, and then sigma comes out 0 and
// the product x * 0 is NaN as well, so the activation's value is the same for
// every input (a finite or infinite z takes the identical sequence).
__device__ __forceinline__ float sigmoid_of(float z)
{
    const float e = exp32_nonpos<false>(-__builtin_fabsf(z));
    const float r = rcp_1_2(1.0f + e);   // 1 + e is in [1, 2]
    return z >= 0.0f ? r : e * r;
}

constexpr float K_SQRT_2_OVER_PI = 0.797884560802865355879892119868763737f;
constexpr float K_CUBIC = 0.044715f;
constexpr float K_CUBIC3 = 0.134145f;
constexpr float K_2SQRT_2_OVER_PI = 1.59576912160573071175978423973752747f;
static_assert(K_2SQRT_2_OVER_PI == 2.0f * K_SQRT_2_OVER_PI, "the doubled constant is exact");

// 2u for u = fl32(sqrt(2/pi) * inner), as one multiply: fl32(2 sqrt(2/pi) *
// inner) equals fl32(u + u) because doubling commutes with rounding, except
// where u is subnormal -- and there both give sigma = 1 - sigma = 1/2, so the
// activations below come out bit-identical to the u + u form.
__device__ __forceinline__ float gelu_2u(float inner) { return K_2SQRT_2_OVER_PI * inner; }

// tanh-form GELU: x * sigma(2u), u = sqrt(2/pi)(x + 0.044715 x^3); this equals
// 0.5 x (1 + tanh u).
__device__ __forceinline__ float gelu32(float x)
{
    float x2 = x * x;
    float x3 = x2 * x;
    float inner = __builtin_fmaf(K_CUBIC, x3, x);
    return x * sigmoid_of(gelu_2u(inner));
}

// d/dx of gelu32's function: sigma + x sigma (1 - sigma) 2u'(x), with
// 2u'(x) = 2 sqrt(2/pi) (1 + 3 * 0.044715 x^2); the second term is 0 when
// sigma(1 - sigma) is 0.
__device__ __forceinline__ float dgelu32(float x)
{
    float x2 = x * x;
    float x3 = x2 * x;
    float inner = __builtin_fmaf(K_CUBIC, x3, x);
    float s, sc;
    sigmoid_pair(gelu_2u(inner), s, sc);
    float ss = s * sc;
    float du = K_2SQRT_2_OVER_PI * __builtin_fmaf(K_CUBIC3, x2, 1.0f);
    float t = ss == 0.0f ? 0.0f : (x * ss) * du;
    return s + t;
}

__device__ __forceinline__ float silu32(float g) { return g * sigmoid_of(g); }

// d/dg of silu32's function: sigma + g sigma (1 - sigma); the second term is
// 0 when sigma(1 - sigma) is 0.
__device__ __forceinline__ float dsilu32(float g)
{
    float s, sc;
    sigmoid_pair(g, s, sc);
    float ss = s * sc;
    float t = ss == 0.0f ? 0.0f : g * ss;
    return s + t;
}

// Gated backward of one element pair: with a = act(gate), da = act'(gate)
// (SiLU for OP_DSWIGLU, GELU for OP_DGEGLU; one shared logistic evaluation,
// the same values as silu32/dsilu32 or gelu32/dgelu32), d_gate =
// (da * grad) * linear and d_linear = a * grad.
template <int OP>
__device__ __forceinline__ float dgated_value(float gate, float grad, float lin, bool gate_half)
{
    float s, sc, a, da;
    if constexpr (OP == OP_DSWIGLU) {
        sigmoid_pair(gate, s, sc);
        a = gate * s;
        float ss = s * sc;
        da = s + (ss == 0.0f ? 0.0f : gate * ss);
    } else {
        float x2 = gate * gate;
        float x3 = x2 * gate;
        float inner = __builtin_fmaf(K_CUBIC, x3, gate);
        sigmoid_pair(gelu_2u(inner), s, sc);
        a = gate * s;
        float ss = s * sc;
        float du = K_2SQRT_2_OVER_PI * __builtin_fmaf(K_CUBIC3, x2, 1.0f);
        da = s + (ss == 0.0f ? 0.0f : (gate * ss) * du);
    }
    if (gate_half) {
        float t = da * grad;
        return t * lin;
    }
    return a * grad;
}

// y (fp32, before the bf16 rounding) for one element.  a = x (or gate),
// b = grad (or linear).
template <int OP>
__device__ __forceinline__ float fused_value(float a, float b)
{
    if constexpr (OP == OP_GELU)
        return gelu32(a);
    else if constexpr (OP == OP_DGELU)
        return dgelu32(a) * b;
    else if constexpr (OP == OP_SWIGLU)
        return silu32(a) * b;
    else if constexpr (OP == OP_DSILU)
        return dsilu32(a) * b;
    else
        return gelu32(a) * b;
}

// Apply the pre-op to a packed pair of bf16 (with its partner pair) and round
// the two results to bf16.
template <int OP>
__device__ __forceinline__ uint32_t fused_pair(uint32_t a, uint32_t b)
{
    return bf16x2_rne(fused_value<OP>(bf16_lo(a), bf16_lo(b)),
                      fused_value<OP>(bf16_hi(a), bf16_hi(b)));
}

// Gated backward of packed pairs (gate, grad, linear words), rounded to bf16.
template <int OP>
__device__ __forceinline__ uint32_t dgated_pair(uint32_t g, uint32_t dy, uint32_t l, bool gate_half)
{
    return bf16x2_rne(dgated_value<OP>(bf16_lo(g), bf16_lo(dy), bf16_lo(l), gate_half),
                      dgated_value<OP>(bf16_hi(g), bf16_hi(dy), bf16_hi(l), gate_half));
}

// ---------------------------------------------------------------------------
// Cross-lane max within aligned groups of 2 / 4 lanes (DPP quad permutes,
// no LDS traffic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t max_xor1(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); // [1,0,3,2]
    return v > o ? v : o;
}
__device__ __forceinline__ uint32_t max_xor2(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false); // [2,3,0,1]
    return v > o ? v : o;
}

// Hardware dispatches workgroup i to XCD (i mod 8).  Give each XCD a
// contiguous range of logical tiles so that neighbouring tiles (which share
// scale-tensor cache lines) are written through the same L2.
__device__ __forceinline__ int xcd_tile(int bid, int nblocks)
{
    int per = nblocks >> 3, rem = nblocks & 7;
    int xcd = bid & 7, slot = bid >> 3;
    return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace mxk
