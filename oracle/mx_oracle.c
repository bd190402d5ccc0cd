/*
 * mx_oracle.c -- CPU oracle for block-scaled quantisation of bf16 tensors
 * (MXFP8: E8M0 scale per 32 elements + E4M3 elements; NVFP4: fp32 tensor
 * scale + E4M3 scale per 16 elements + E2M1 elements).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code, header, table or constant with the HIP library and
 * includes nothing from it.
 *
 * Style: every value is decoded from its bit pattern with the format's own
 * definition, held exactly in a double, and every encoder searches for the
 * nearest representable value of the target format.  No bit tricks, no
 * blocking, no fusion.  Where the method fixes fp32 arithmetic (the fused
 * activations and the NVFP4 scale chain) the step is written as an explicit
 * fp32 operation; "fl32(a op b)" below is computed as (float)((double)a op b),
 * which is the correctly rounded fp32 result because a double carries more
 * than 2*24+2 bits (double rounding is innocuous for + - * /).
 *
 * Sources.  The pages ("[Common] Fix pointer arithmatic to generate correct
 * LDS/STS instructions", TransformerEngine PR 3291; "Multiply with inverse
 * scale in loop inside of dividing to improve perf", torchao PR 12) name the
 * MXFP8 / NVFP4 cast kernels and their fusions (tables "MXFP8 generic quantize
 * kernel", "MXFP8 gated (swiglu / geglu) kernel", "NVFP4 2D quantize-transpose
 * kernel") but never define the arithmetic.  The rules below are the readings
 * this oracle implements:
 *   R1  E8M0 shared exponent = floor(log2(amax)) - 8 (8 = exponent of the
 *       largest E4M3 binade), biased by 127 and clamped to [0, 254].
 *   R2  element = E4M3(x / 2^(byte-127)), round to nearest, ties to the even
 *       code, magnitudes above 448 saturate to 448, sign kept (-0 -> 0x80).
 *   R3  a block holding Inf or NaN gets scale 0xFF and elements 0x7F.
 *   R4  column-wise output is the row-wise output of the transpose.
 *   R5  fused pre-ops are evaluated in fp32 by the sequences in this file and
 *       rounded once to bf16 (RNE); that bf16 tensor is what gets quantised
 *       and what dbias sums.  The backward ones (dSiLU, dSwiGLU, dGeGLU, named
 *       in the "MXFP8 generic quantize kernel" and gated tables) use the
 *       derivative of the same forward sequences, in the order written in
 *       orc_preop() and orc_gated_bwd().
 *   R6  NVFP4 per the chain in nvfp4_block(), with the tensor amax A the
 *       largest |x| (NaN if an element is NaN, else Inf if one is infinite).
 *       A tensor whose A is not finite has no usable global scale: its scale
 *       bytes are 0x7F (the E4M3 NaN), its element codes 0, and S_g =
 *       fl32(A / 2688) stays Inf or NaN.
 *   R7  format variants (flags beside the axis bits): E5M2 elements (bias 15,
 *       max 57344, emax 15) in place of E4M3, and the round-up scale rule,
 *       byte = ceil(log2(amax / max_elem)) + 127: the smallest power of two
 *       that brings amax inside the element range, so nothing saturates.
 *       The floor rule of R1 reads emax = 15 for E5M2.
 *   R8  GEMM-ready scale layout (flag beside the axis bits): the scales of a
 *       [R][C] scale matrix are regrouped into tiles of 32 rows x 8 blocks,
 *       one per wave step group of a 32x32x64 block-scaled MFMA: inside a
 *       tile, the 4-byte word of lane L holds, in byte j, the scale that lane
 *       uses in the j-th of four consecutive K steps (row L % 32, block
 *       2j + L / 32).  Tiles are stored block-tile-major; R and C are padded
 *       to whole tiles with zero bytes.
 *   R10 grouped cast: groups stacked along rows, each cast as a tensor of its
 *       own, outputs concatenated group after group.
 *   R9  a line whose length is not a multiple of 32 ends in a partial block:
 *       its scale and codes come from its own elements alone (the same as
 *       padding the line with zeros, which never change an amax and encode
 *       to zero).  NVFP4 likewise for lines that are not multiples of 16
 *       (2D: partial 16 x 16 blocks at the edges); a line of n codes packs
 *       into ceil(n/2) bytes, the high nibble of the last one 0 when n is
 *       odd -- again the zero-padded tensor's bytes.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * -fPIC (see build.py).  OpenMP only splits independent rows / columns /
 * blocks, never a reduction, so results do not depend on the thread count.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_SHAPE 3
#define ORC_ERR_ENUM 2
#define ORC_ERR_NOMEM 9

/* ------------------------------------------------------------------------ */
/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits.        */
/* ------------------------------------------------------------------------ */

double orc_bf16_value(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -133);           /* (m/128) * 2^-126 */
    else
        mag = ldexp(128.0 + m, e - 134);        /* (1 + m/128) * 2^(e-127) */
    return s ? -mag : mag;
}

/* Nearest bf16 to v, ties to the even significand, overflow to Inf. */
uint16_t orc_bf16_round(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                   /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                  /* floor(log2 a) */
    if (e < -126)
        e = -126;                    /* subnormals share the last binade's spacing */
    double q = ldexp(1.0, e - 7);    /* bf16 spacing in this binade */
    double n = nearbyint(a / q);     /* default rounding mode: nearest, ties even */
    double r = n * q;
    if (r >= 0x1p128)
        return sign | 0x7F80;
    if (r < 0x1p-126)
        return sign | (uint16_t)(r / 0x1p-133);
    frexp(r, &ex);
    e = ex - 1;
    int m = (int)(r / ldexp(1.0, e - 7)) - 128;
    return sign | (uint16_t)((e + 127) << 7) | (uint16_t)m;
}

/* ------------------------------------------------------------------------ */
/* E4M3 ("fn" variant): bias 7, no Inf, 0x7F / 0xFF are NaN, max 448.         */
/* ------------------------------------------------------------------------ */

double orc_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);             /* (m/8) * 2^-6 */
    else
        mag = ldexp(8.0 + m, e - 10);           /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

static double E4M3_MAG[127];   /* magnitudes of codes 0x00..0x7E, increasing */
static double E2M1_MAG[8];     /* magnitudes of codes 0x0..0x7, increasing */
static double E5M2_MAG[124];
double orc_e5m2_value(uint8_t c);

double orc_e2m1_value(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m                       /* subnormal: m/2 */
                          : ldexp(1.0 + 0.5 * m, e - 1);  /* (1 + m/2) * 2^(e-1) */
    return s ? -mag : mag;
}

static void init_tables(void)
{
    static int done = 0;
    if (done)
        return;
    for (int c = 0; c < 127; c++)
        E4M3_MAG[c] = orc_e4m3_value((uint8_t)c);
    for (int c = 0; c < 8; c++)
        E2M1_MAG[c] = orc_e2m1_value((uint8_t)c);
    for (int c = 0; c < 124; c++)
        E5M2_MAG[c] = orc_e5m2_value((uint8_t)c);
    done = 1;
}

void orc_init(void) { init_tables(); }

/* Nearest of the magnitudes mag[0..n-1] (increasing) to a >= 0, a < mag[n-1];
 * on a tie the even code wins. */
static int nearest_code(const double *mag, int n, double a)
{
    int lo = 0, hi = n - 1;       /* mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (mag[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - mag[lo], dhi = mag[hi] - a;
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1) ? hi : lo;
}

/* R2: round to nearest E4M3, ties to even code, saturate at 448, keep sign. */
uint8_t orc_e4m3_encode(double v)
{
    init_tables();
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E;
    return sign | (uint8_t)nearest_code(E4M3_MAG, 127, a);
}

/* E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; nearest, ties to even code,
 * saturate at 6 (Inf included), sign in bit 3, NaN -> +0. */
uint8_t orc_e2m1_encode(double v)
{
    init_tables();
    if (isnan(v))
        return 0x0;
    uint8_t sign = signbit(v) ? 0x8 : 0;
    double a = fabs(v);
    if (a >= 6.0)
        return sign | 0x7;
    return sign | (uint8_t)nearest_code(E2M1_MAG, 8, a);
}

/* ------------------------------------------------------------------------ */
/* E5M2: bias 15, 0x7C = Inf, 0x7D..0x7F NaN, max finite 57344 (0x7B).        */
/* ------------------------------------------------------------------------ */

double orc_e5m2_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 0x1F, m = c & 3;
    double mag;
    if (e == 31)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -16);            /* (m/4) * 2^-14 */
    else
        mag = ldexp(4.0 + m, e - 17);           /* (1 + m/4) * 2^(e-15) */
    return s ? -mag : mag;
}

/* E5M2_MAG: magnitudes of codes 0x00..0x7B, increasing. */

/* Nearest E5M2, ties to even code, saturating at 57344 (Inf included: the
 * saturating conversion never makes Inf), sign kept, NaN -> 0x7F. */
uint8_t orc_e5m2_encode(double v)
{
    init_tables();
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 57344.0)
        return sign | 0x7B;
    return sign | (uint8_t)nearest_code(E5M2_MAG, 124, a);
}

/* ------------------------------------------------------------------------ */
/* E8M0 shared scale (R1).                                                   */
/* ------------------------------------------------------------------------ */

double orc_e8m0_value(uint8_t b)
{
    return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127);
}

uint8_t orc_e8m0_byte(double amax)
{
    if (isnan(amax) || isinf(amax))
        return 0xFF;
    if (amax == 0.0)
        return 0;
    int ex;
    frexp(amax, &ex);                  /* floor(log2 amax) = ex - 1 */
    int b = (ex - 1) - 8 + 127;        /* E4M3's largest binade is 2^8 */
    if (b < 0)
        b = 0;
    if (b > 254)
        b = 254;
    return (uint8_t)b;
}

/* Element formats of an MX block (R7): exponent of the largest binade and
 * the largest finite magnitude. */
#define ORC_E5M2 4u        /* flag: E5M2 elements */
#define ORC_ROUND_UP 8u    /* flag: round-up scale rule */

static int fmt_emax(unsigned mode) { return (mode & ORC_E5M2) ? 15 : 8; }
static double fmt_max(unsigned mode) { return (mode & ORC_E5M2) ? 57344.0 : 448.0; }

/* E8M0 byte of a block under either rule (R1 / R7).
 *   floor:    floor(log2 amax) - emax
 *   round up: the smallest integer t with amax <= max_elem * 2^t,
 *             i.e. ceil(log2(amax / max_elem)), found by counting up from a
 *             value known to be too small (every comparison is exact).
 * Biased by 127 and clamped to [0, 254]; amax = 0 -> 0; Inf / NaN -> 0xFF. */
uint8_t orc_e8m0_byte_mode(double amax, unsigned mode)
{
    if (isnan(amax) || isinf(amax))
        return 0xFF;
    if (amax == 0.0)
        return 0;
    int ex;
    frexp(amax, &ex);                  /* floor(log2 amax) = ex - 1 */
    int t;
    if (mode & ORC_ROUND_UP) {
        t = (ex - 1) - fmt_emax(mode) - 1;     /* max * 2^t < 2^(ex-1) <= amax */
        while (amax > ldexp(fmt_max(mode), t))
            t++;
    } else {
        t = (ex - 1) - fmt_emax(mode);
    }
    int b = t + 127;
    if (b < 0)
        b = 0;
    if (b > 254)
        b = 254;
    return (uint8_t)b;
}

/* One MX block: n values (exact doubles) -> n element codes (q[i*qstride])
 * and the E8M0 byte; mode selects the element format and the scale rule (R7).
 * The scale is applied as a true division by 2^(byte-127); that is exact
 * here, so it equals multiplying by the power-of-two inverse (the point of
 * "Multiply with inverse scale in loop inside of dividing", body bullets). */
void orc_mx_block_mode(const double *v, int n, uint8_t *q, int64_t qstride, uint8_t *s,
                       unsigned mode)
{
    double amax = 0.0;
    int nonfinite = 0;
    for (int i = 0; i < n; i++) {
        if (!isfinite(v[i]))
            nonfinite = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    if (nonfinite) {                               /* R3 */
        *s = 0xFF;
        for (int i = 0; i < n; i++)
            q[i * qstride] = 0x7F;
        return;
    }
    uint8_t b = orc_e8m0_byte_mode(amax, mode);
    double X = orc_e8m0_value(b);
    for (int i = 0; i < n; i++)
        q[i * qstride] = (mode & ORC_E5M2) ? orc_e5m2_encode(v[i] / X)
                                           : orc_e4m3_encode(v[i] / X);
    *s = b;
}

/* The default block: E4M3 elements, floor rule (R1, R2). */
void orc_mx_block(const double *v, int n, uint8_t *q, int64_t qstride, uint8_t *s)
{
    orc_mx_block_mode(v, n, q, qstride, s, 0u);
}

/* ------------------------------------------------------------------------ */
/* Fused pre-op arithmetic (R5).  Every line is one IEEE fp32 operation;     */
/* fmaf is the fused multiply-add with a single rounding.                    */
/* ------------------------------------------------------------------------ */

/* e^a in fp32: Cody & Waite argument reduction a = n*ln2 + r with ln2 split
 * as 355/512 + (ln2 - 355/512), then the degree-7 Taylor polynomial of e^r
 * (|r| <= ln2/2) evaluated by Horner with fmaf, then scaling by 2^n as two
 * exact power-of-two factors so that subnormal results round once. */
float orc_exp32(float a)
{
    const float LOG2E = 1.44269504088896340736f;       /* 1/ln 2 */
    const float LN2_HI = 0.693359375f;                 /* 355/512, exact */
    const float LN2_LO = -2.12194440054690583e-4f;     /* ln 2 - 355/512 */
    const float C2 = 1.0f / 2.0f, C3 = (float)(1.0 / 6.0), C4 = (float)(1.0 / 24.0),
                C5 = (float)(1.0 / 120.0), C6 = (float)(1.0 / 720.0),
                C7 = (float)(1.0 / 5040.0);
    if (a != a)
        return a;
    if (a > 88.72283172607421875f)      /* e^a would round to +Inf */
        return INFINITY;
    if (a < -104.0f)                    /* e^a below half the least subnormal */
        return 0.0f;
    float n = rintf(a * LOG2E);
    float r = fmaf(n, -LN2_HI, a);
    r = fmaf(n, -LN2_LO, r);
    float p = C7;
    p = fmaf(p, r, C6);
    p = fmaf(p, r, C5);
    p = fmaf(p, r, C4);
    p = fmaf(p, r, C3);
    p = fmaf(p, r, C2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;                    /* in [-150, 128] */
    int n1 = ni / 2, n2 = ni - n1;      /* each in [-75, 64]: 2^n1, 2^n2 are normal */
    return (p * ldexpf(1.0f, n1)) * ldexpf(1.0f, n2);
}

/* Logistic sigma(z) = 1/(1+e^-z) and its complement 1 - sigma(z), both built
 * from e = e^-|z| <= 1 so that nothing overflows and neither is computed by
 * cancellation:  for z >= 0: sigma = 1/(1+e), 1-sigma = e/(1+e); for z < 0
 * the two swap. */
static void sigmoid_pair(float z, float *s, float *sc)
{
    float e = orc_exp32(-fabsf(z));
    float d = 1.0f + e;
    float r = 1.0f / d;
    float er = e * r;
    if (z >= 0.0f) {
        *s = r;
        *sc = er;
    } else {
        *s = er;
        *sc = r;
    }
}

static const float GELU_K0 = 0.797884560802865355879892119868763737f;  /* sqrt(2/pi) */
static const float GELU_K1 = 0.044715f;
static const float GELU_K3 = 0.134145f;                                 /* 3 * 0.044715 */
static const float GELU_2K0 = 1.59576912160573071175978423973752747f;  /* 2*sqrt(2/pi) */

/* tanh-form GELU: 0.5*x*(1 + tanh(u)), u = sqrt(2/pi)*(x + 0.044715 x^3),
 * evaluated through the identity 0.5*(1 + tanh(u)) = sigma(2u). */
float orc_gelu32(float x)
{
    float x2 = x * x;
    float x3 = x2 * x;
    float inner = fmaf(GELU_K1, x3, x);
    float u = GELU_K0 * inner;
    float s, sc;
    sigmoid_pair(u + u, &s, &sc);
    return x * s;
}

/* d/dx of the GELU above: sigma(2u) + x * sigma(2u)(1 - sigma(2u)) * 2u'(x),
 * 2u'(x) = 2*sqrt(2/pi)*(1 + 3*0.044715 x^2).  When sigma(1-sigma) is 0 the
 * second term is 0 (this also keeps 0 * Inf out for huge |x|). */
float orc_dgelu32(float x)
{
    float x2 = x * x;
    float x3 = x2 * x;
    float inner = fmaf(GELU_K1, x3, x);
    float u = GELU_K0 * inner;
    float s, sc;
    sigmoid_pair(u + u, &s, &sc);
    float ss = s * sc;
    float du = GELU_2K0 * fmaf(GELU_K3, x2, 1.0f);
    float t = (ss == 0.0f) ? 0.0f : (x * ss) * du;
    return s + t;
}

/* SiLU: g * sigma(g). */
float orc_silu32(float g)
{
    float s, sc;
    sigmoid_pair(g, &s, &sc);
    return g * s;
}

/* d/dg of the SiLU above: sigma(g) + g * sigma(g)(1 - sigma(g)); the second
 * term is 0 when sigma(1 - sigma) is 0 (as for dGELU). */
float orc_dsilu32(float g)
{
    float s, sc;
    sigmoid_pair(g, &s, &sc);
    float ss = s * sc;
    float t = (ss == 0.0f) ? 0.0f : g * ss;
    return s + t;
}

static float f32_of_bf16(uint16_t b) { return (float)orc_bf16_value(b); }

/* The fused elementwise value y (as bf16 bits) for one input element.
 * pre: 0 none, 1 GELU(x), 2 dGELU(x) * grad, 3 dSiLU(x) * grad. */
uint16_t orc_preop(int pre, uint16_t x, uint16_t grad)
{
    switch (pre) {
    case 3: {
        float d = orc_dsilu32(f32_of_bf16(x));
        float y = d * f32_of_bf16(grad);
        return orc_bf16_round(y);
    }
    case 0:
        return x;
    case 1:
        return orc_bf16_round(orc_gelu32(f32_of_bf16(x)));
    case 2: {
        float d = orc_dgelu32(f32_of_bf16(x));
        float y = d * f32_of_bf16(grad);
        return orc_bf16_round(y);
    }
    default:
        return 0x7FC0;
    }
}

/* Gated value for one output element. act: 1 SwiGLU, 2 GeGLU. */
uint16_t orc_gated(int act, uint16_t gate, uint16_t lin)
{
    float g = f32_of_bf16(gate), l = f32_of_bf16(lin);
    float a;
    if (act == 1)
        a = orc_silu32(g);
    else if (act == 2)
        a = orc_gelu32(g);
    else
        return 0x7FC0;
    float y = a * l;
    return orc_bf16_round(y);
}

/* Gated backward for one element pair: with a = act(gate), da = act'(gate)
 * (act 1 SiLU, 2 GELU), the gradients of the two input halves are
 *   d_gate = fl32(fl32(da * grad) * linear),   d_lin = fl32(a * grad),
 * each rounded once to bf16. */
int orc_gated_bwd(int act, uint16_t gate, uint16_t lin, uint16_t grad, uint16_t *d_gate,
                  uint16_t *d_lin)
{
    float g = f32_of_bf16(gate), l = f32_of_bf16(lin), dy = f32_of_bf16(grad);
    float a, da;
    if (act == 1) {
        a = orc_silu32(g);
        da = orc_dsilu32(g);
    } else if (act == 2) {
        a = orc_gelu32(g);
        da = orc_dgelu32(g);
    } else {
        return ORC_ERR_ENUM;
    }
    float t = da * dy;
    float yg = t * l;
    float yl = a * dy;
    *d_gate = orc_bf16_round(yg);
    *d_lin = orc_bf16_round(yl);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* GEMM-ready scale layout (R8).                                             */
/* ------------------------------------------------------------------------ */

#define ORC_TILED 16u      /* flag: scales in the MFMA tile layout */

/* Bytes of the tiled form of an R x C scale matrix. */
int64_t orc_tiled_scale_bytes(int64_t R, int64_t C)
{
    return ((R + 31) / 32) * ((C + 7) / 8) * 256;
}

/* Compact row-major scales s[R][C] -> the tile layout.  A 32x32x64 MFMA step
 * with block-scaled operands has lane L hold one row (L % 32) and one block of
 * 32 K elements (the first or second half of the step's 64, by L / 32), and
 * takes its scale from a byte of a 32-bit register chosen per step.  So the
 * scales a wave needs for four consecutive steps (8 blocks of 32 rows) form a
 * 256-byte tile in which lane L's word holds its scale for step j in byte j:
 * block 2j + L / 32 of row L % 32.  Tile (row tile rt, block tile bt) sits at
 * (bt * RT + rt) * 256, RT = ceil(R / 32); bytes outside the matrix are 0. */
void orc_scale_tiles(const uint8_t *s, int64_t R, int64_t C, uint8_t *out)
{
    const int64_t RT = (R + 31) / 32;
    memset(out, 0, (size_t)orc_tiled_scale_bytes(R, C));
    for (int64_t r = 0; r < R; r++)
        for (int64_t c = 0; c < C; c++) {
            const int64_t tile = (c / 8) * RT + r / 32;
            const int64_t lane = 32 * (c % 2) + r % 32;
            const int64_t step = (c % 8) / 2;
            out[tile * 256 + 4 * lane + step] = s[r * C + c];
        }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 over a tensor.                                                      */
/* ------------------------------------------------------------------------ */

/* Blocks of 32 along a line of n elements; the last one is partial when 32
 * does not divide n (R9). */
static int64_t nblocks(int64_t n) { return (n + 31) / 32; }

/* Row-wise and column-wise MX quantisation of the bf16 tensor y[M][K].
 *   rows: q_row[M][K], s_row[M][ceil(K/32)]   (blocks of 32 along K)
 *   cols: q_col[K][M], s_col[K][ceil(M/32)]   (blocks of 32 along M, stored
 *         as the row-wise output of the transpose, R4)
 * A block at the end of a line that has fewer than 32 elements is quantised
 * from those elements alone (R9).
 * axis bits 0, 1 select the outputs; ORC_E5M2 / ORC_ROUND_UP the variant. */
static void mx_tensor(const uint16_t *y, int64_t M, int64_t K, unsigned axis,
                      uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col)
{
    if (axis & 1u) {
        const int64_t nb = nblocks(K);
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; m++) {
            double v[32];
            for (int64_t j = 0; j < nb; j++) {
                const int n = (int)(K - 32 * j < 32 ? K - 32 * j : 32);
                for (int i = 0; i < n; i++)
                    v[i] = orc_bf16_value(y[m * K + 32 * j + i]);
                orc_mx_block_mode(v, n, q_row + m * K + 32 * j, 1, s_row + m * nb + j, axis);
            }
        }
    }
    if (axis & 2u) {
        const int64_t nb = nblocks(M);
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < K; k++) {
            double v[32];
            for (int64_t j = 0; j < nb; j++) {
                const int n = (int)(M - 32 * j < 32 ? M - 32 * j : 32);
                for (int i = 0; i < n; i++)
                    v[i] = orc_bf16_value(y[(32 * j + i) * K + k]);
                orc_mx_block_mode(v, n, q_col + k * M + 32 * j, 1, s_col + k * nb + j, axis);
            }
        }
    }
}

/* mx_tensor with the scales in the layout the axis flags ask for: compact
 * [rows][blocks], or (ORC_TILED) the tile layout of R8. */
static int mx_tensor_out(const uint16_t *y, int64_t M, int64_t K, unsigned axis,
                         uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col)
{
    if (!(axis & ORC_TILED)) {
        mx_tensor(y, M, K, axis, q_row, s_row, q_col, s_col);
        return ORC_OK;
    }
    uint8_t *sr = (axis & 1u) ? (uint8_t *)malloc((size_t)(M * nblocks(K))) : NULL;
    uint8_t *sc = (axis & 2u) ? (uint8_t *)malloc((size_t)(K * nblocks(M))) : NULL;
    if (((axis & 1u) && !sr) || ((axis & 2u) && !sc)) {
        free(sr);
        free(sc);
        return ORC_ERR_NOMEM;
    }
    mx_tensor(y, M, K, axis, q_row, sr, q_col, sc);
    if (sr)
        orc_scale_tiles(sr, M, nblocks(K), s_row);
    if (sc)
        orc_scale_tiles(sc, K, nblocks(M), s_col);
    free(sr);
    free(sc);
    return ORC_OK;
}

/* dbias[k] = sum over m of y[m][k]: summed in double in row order, rounded
 * once to fp32. */
static void column_sums(const uint16_t *y, int64_t M, int64_t K, float *dbias)
{
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; k++) {
        double acc = 0.0;
        for (int64_t m = 0; m < M; m++)
            acc += orc_bf16_value(y[m * K + k]);
        dbias[k] = (float)acc;
    }
}

/* axis: bit 0 rows, bit 1 columns, ORC_E5M2 / ORC_ROUND_UP variants (R7),
 * ORC_TILED scale layout (R8: s_row / s_col then hold the tiled bytes).
 * fusion: low nibble = pre-op (0 none, 1 GELU, 2 dGELU, 3 dSiLU), bit 0x10 = dbias.
 * y_out (optional, [M][K]) receives the fused bf16 tensor. */
int orc_mx_quantize(const uint16_t *x, const uint16_t *grad, int64_t M, int64_t K,
                    unsigned axis, int fusion, uint8_t *q_row, uint8_t *s_row,
                    uint8_t *q_col, uint8_t *s_col, float *dbias, uint16_t *y_out)
{
    int pre = fusion & 0xF;
    if (M <= 0 || K <= 0)
        return ORC_ERR_SHAPE;
    if (pre > 3 || (fusion & ~0x1F) || (axis & ~31u))
        return ORC_ERR_ENUM;
    init_tables();
    const uint16_t *y = x;
    uint16_t *ybuf = NULL;
    if (pre != 0) {
        ybuf = y_out ? y_out : (uint16_t *)malloc((size_t)(M * K) * 2);
        if (!ybuf)
            return ORC_ERR_NOMEM;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M * K; i++)
            ybuf[i] = orc_preop(pre, x[i], grad ? grad[i] : 0);
        y = ybuf;
    } else if (y_out) {
        memcpy(y_out, x, (size_t)(M * K) * 2);
    }
    int rc = mx_tensor_out(y, M, K, axis, q_row, s_row, q_col, s_col);
    if (rc == ORC_OK && (fusion & 0x10) && dbias)
        column_sums(y, M, K, dbias);
    if (ybuf && ybuf != y_out)
        free(ybuf);
    return rc;
}

/* x[M][2N] = [gate | linear] (gate = columns 0..N-1); y[m][n] = act(gate)*lin. */
int orc_mx_quantize_gated(const uint16_t *x, int64_t M, int64_t N, unsigned axis, int act,
                          uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                          uint16_t *y_out)
{
    if (M <= 0 || N <= 0)
        return ORC_ERR_SHAPE;
    if ((act != 1 && act != 2) || (axis & ~31u))
        return ORC_ERR_ENUM;
    init_tables();
    uint16_t *y = y_out ? y_out : (uint16_t *)malloc((size_t)(M * N) * 2);
    if (!y)
        return ORC_ERR_NOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = orc_gated(act, x[m * 2 * N + n], x[m * 2 * N + N + n]);
    int rc = mx_tensor_out(y, M, N, axis, q_row, s_row, q_col, s_col);
    if (y != y_out)
        free(y);
    return rc;
}

/* Gated backward cast: grad[M][N], x[M][2N] = [gate | linear]; the tensor
 * quantised is dx[M][2N] = [d_gate | d_lin] (orc_gated_bwd per element). */
int orc_mx_quantize_dgated(const uint16_t *grad, const uint16_t *x, int64_t M, int64_t N,
                           unsigned axis, int act, uint8_t *q_row, uint8_t *s_row,
                           uint8_t *q_col, uint8_t *s_col, uint16_t *y_out)
{
    if (M <= 0 || N <= 0)
        return ORC_ERR_SHAPE;
    if ((act != 1 && act != 2) || (axis & ~31u))
        return ORC_ERR_ENUM;
    init_tables();
    uint16_t *y = y_out ? y_out : (uint16_t *)malloc((size_t)(M * 2 * N) * 2);
    if (!y)
        return ORC_ERR_NOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            orc_gated_bwd(act, x[m * 2 * N + n], x[m * 2 * N + N + n], grad[m * N + n],
                          &y[m * 2 * N + n], &y[m * 2 * N + N + n]);
    int rc = mx_tensor_out(y, M, 2 * N, axis, q_row, s_row, q_col, s_col);
    if (y != y_out)
        free(y);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Grouped (per-expert) MXFP8 cast (R10).                                    */
/* ------------------------------------------------------------------------ */

/* Bytes of one scale tensor of a [rows][cols] cast blocked along cols, in the
 * layout the axis flags ask for. */
static int64_t scale_bytes(int64_t rows, int64_t cols, unsigned axis)
{
    if (rows == 0)
        return 0;
    return (axis & ORC_TILED) ? orc_tiled_scale_bytes(rows, nblocks(cols)) : rows * nblocks(cols);
}

/* G tensors stacked along rows: x[M][K] with group g owning rows
 * [r_g, r_g + rows[g]), M = sum of rows[g] (a group may be empty).  Each group
 * is cast exactly as orc_mx_quantize casts a tensor of its own; the outputs
 * are the groups' outputs one after the other:
 *   q_row[M][K]; s_row: group g's scales at sum_{h<g} bytes(rows[h], K);
 *   q_col: group g's [K][rows[g]] at byte K * r_g;
 *   s_col: group g's scales at sum_{h<g} bytes(K, rows[h]);
 *   dbias[G][K]: group g's column sums (0 for an empty group). */
int orc_mx_quantize_grouped(const uint16_t *x, const uint16_t *grad, int64_t K,
                            const int64_t *rows, int G, unsigned axis, int fusion,
                            uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                            float *dbias)
{
    if (G <= 0 || K <= 0)
        return ORC_ERR_SHAPE;
    int64_t r = 0, sr = 0, sc = 0;
    for (int g = 0; g < G; g++) {
        const int64_t m = rows[g];
        if (m < 0)
            return ORC_ERR_SHAPE;
        if (m > 0) {
            int rc = orc_mx_quantize(x + r * K, grad ? grad + r * K : NULL, m, K, axis, fusion,
                                     q_row ? q_row + r * K : NULL, s_row ? s_row + sr : NULL,
                                     q_col ? q_col + K * r : NULL, s_col ? s_col + sc : NULL,
                                     dbias ? dbias + (int64_t)g * K : NULL, NULL);
            if (rc != ORC_OK)
                return rc;
        } else if (dbias && (fusion & 0x10)) {
            for (int64_t k = 0; k < K; k++)
                dbias[(int64_t)g * K + k] = 0.0f;
        }
        sr += scale_bytes(m, K, axis);
        sc += scale_bytes(K, m, axis);
        r += m;
    }
    return ORC_OK;
}

/* Grouped gated casts (R10): x[M][2N] = [gate | linear] rows stacked by group;
 * group g's output tensor is that of orc_mx_quantize_gated (forward, grad
 * NULL: y[rows][N]) or orc_mx_quantize_dgated (backward: grad[M][N] given,
 * dx[rows][2N]); outputs concatenated group after group as in
 * orc_mx_quantize_grouped, with W = N (forward) or 2N (backward) the width of
 * the quantised tensor. */
int orc_mx_quantize_gated_grouped(const uint16_t *grad, const uint16_t *x, int64_t N,
                                  const int64_t *rows, int G, unsigned axis, int act,
                                  uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col)
{
    if (G <= 0 || N <= 0)
        return ORC_ERR_SHAPE;
    const int64_t W = grad ? 2 * N : N;
    int64_t r = 0, sr = 0, sc = 0;
    for (int g = 0; g < G; g++) {
        const int64_t m = rows[g];
        if (m < 0)
            return ORC_ERR_SHAPE;
        if (m > 0) {
            uint8_t *qr = q_row ? q_row + r * W : NULL, *srp = s_row ? s_row + sr : NULL;
            uint8_t *qc = q_col ? q_col + W * r : NULL, *scp = s_col ? s_col + sc : NULL;
            int rc = grad ? orc_mx_quantize_dgated(grad + r * N, x + r * 2 * N, m, N, axis, act,
                                                   qr, srp, qc, scp, NULL)
                          : orc_mx_quantize_gated(x + r * 2 * N, m, N, axis, act, qr, srp, qc,
                                                  scp, NULL);
            if (rc != ORC_OK)
                return rc;
        }
        sr += scale_bytes(m, W, axis);
        sc += scale_bytes(W, m, axis);
        r += m;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 (R6).                                                               */
/* ------------------------------------------------------------------------ */

/* Largest magnitude of the tensor, as the (exact) fp32 value; NaN when an
 * element is NaN (a NaN has no magnitude to compare), +Inf when one is
 * infinite and none is NaN. */
float orc_absmax(const uint16_t *x, int64_t n)
{
    double a = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double v = fabs(orc_bf16_value(x[i]));
        if (v != v)
            return NAN;
        if (v > a)
            a = v;
    }
    return (float)a;
}

/* A tensor whose amax A is not finite (it holds an Inf or a NaN) has no
 * usable global scale (S_g = fl32(A / 2688) is Inf or NaN): every scale byte
 * is 0x7F, the E4M3 NaN, and every element code 0 (R6). */
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void nvfp4_nonfinite(int64_t M, int64_t K, unsigned axis, uint8_t *q_row, uint8_t *s_row,
                            uint8_t *q_col, uint8_t *s_col)
{
    if (axis & 1u) {
        memset(q_row, 0, (size_t)(M * cdiv(K, 2)));
        memset(s_row, 0x7F, (size_t)(M * cdiv(K, 16)));
    }
    if (axis & 2u) {
        memset(q_col, 0, (size_t)(K * cdiv(M, 2)));
        memset(s_col, 0x7F, (size_t)(K * cdiv(M, 16)));
    }
}

/* n codes c[0], c[stride], ... of a line -> ceil(n/2) bytes at q: code 2i in
 * the low nibble of byte i, code 2i+1 in the high nibble (0 past the end). */
static void pack_codes(const uint8_t *c, int n, int stride, uint8_t *q)
{
    for (int i = 0; 2 * i < n; i++)
        q[i] = (uint8_t)(c[2 * i * stride] | (2 * i + 1 < n ? c[(2 * i + 1) * stride] << 4 : 0));
}

/* Tensor scale S_g = fl32(A / (448*6)), or 1 when A = 0. */
float orc_nvfp4_global_scale(float A)
{
    if (A == 0.0f)
        return 1.0f;
    return (float)((double)A / 2688.0);
}

/* One NVFP4 block of n values (exact doubles) with tensor scale Sg:
 *   b    = max |x_i|
 *   s_q  = fl32(fl32(b / 6) / Sg)           block scale relative to Sg
 *   byte = E4M3(s_q)                        stored scale (RNE, saturating)
 *   den  = fl32(decode(byte) * Sg)          the block's effective scale
 *   inv  = den == 0 ? 0 : fl32(1 / den)     one division per block
 *   q_i  = E2M1(fl32(x_i * inv))            one multiply per element
 * Codes are written one per byte into nib[i*stride]; the caller packs. */
static void nvfp4_block(const double *v, int n, float Sg, uint8_t *nib, int64_t stride,
                        uint8_t *s)
{
    double b = 0.0;
    for (int i = 0; i < n; i++)
        if (fabs(v[i]) > b)
            b = fabs(v[i]);
    float b6 = (float)(b / 6.0);
    float sq = (float)((double)b6 / (double)Sg);
    uint8_t sb = orc_e4m3_encode(sq);
    float d = (float)orc_e4m3_value(sb);
    float den = (float)((double)d * (double)Sg);
    float inv = (den == 0.0f) ? 0.0f : (float)(1.0 / (double)den);
    for (int i = 0; i < n; i++) {
        float vs = (float)(v[i] * (double)inv);
        nib[i * stride] = orc_e2m1_encode(vs);
    }
    *s = sb;
}

/* Row-wise NVFP4 of x[M][K] (blocks of 16 along K, the last one partial when
 * 16 does not divide K) into q_row[M][ceil(K/2)] (code of element 2j in the
 * low nibble of byte j, 2j+1 in the high nibble) and s_row[M][ceil(K/16)];
 * and the same for the transpose into q_col[K][ceil(M/2)],
 * s_col[K][ceil(M/16)].  tensor_amax < 0 means "compute it from x"; a NaN or
 * infinite tensor_amax (the amax of a tensor holding a NaN or an Inf) gives
 * the outputs of nvfp4_nonfinite. */
int orc_nvfp4_quantize_transpose(const uint16_t *x, int64_t M, int64_t K, unsigned axis,
                                 float tensor_amax, uint8_t *q_row, uint8_t *s_row,
                                 uint8_t *q_col, uint8_t *s_col, float *sg_out)
{
    if (M <= 0 || K <= 0)
        return ORC_ERR_SHAPE;
    if (axis & ~3u)
        return ORC_ERR_ENUM;
    init_tables();
    float A = tensor_amax < 0.0f ? orc_absmax(x, M * K) : tensor_amax;
    float Sg = orc_nvfp4_global_scale(A);
    if (sg_out)
        *sg_out = Sg;
    if (!isfinite(A)) {
        nvfp4_nonfinite(M, K, axis, q_row, s_row, q_col, s_col);
        return ORC_OK;
    }
    if (axis & 1u) {
        const int64_t nb = cdiv(K, 16), lb = cdiv(K, 2);
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; m++) {
            double v[16];
            uint8_t c[16];
            for (int64_t j = 0; j < nb; j++) {
                const int n = (int)(K - 16 * j < 16 ? K - 16 * j : 16);
                for (int i = 0; i < n; i++)
                    v[i] = orc_bf16_value(x[m * K + 16 * j + i]);
                nvfp4_block(v, n, Sg, c, 1, s_row + m * nb + j);
                pack_codes(c, n, 1, q_row + m * lb + 8 * j);
            }
        }
    }
    if (axis & 2u) {
        const int64_t nb = cdiv(M, 16), lb = cdiv(M, 2);
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < K; k++) {
            double v[16];
            uint8_t c[16];
            for (int64_t j = 0; j < nb; j++) {
                const int n = (int)(M - 16 * j < 16 ? M - 16 * j : 16);
                for (int i = 0; i < n; i++)
                    v[i] = orc_bf16_value(x[(16 * j + i) * K + k]);
                nvfp4_block(v, n, Sg, c, 1, s_col + k * nb + j);
                pack_codes(c, n, 1, q_col + k * lb + 8 * j);
            }
        }
    }
    return ORC_OK;
}

/* NVFP4 with 2D scaling ("nvfp42d" in the quantize-transpose table): one
 * E4M3 scale per 16 x 16 block of x (partial blocks at the right and bottom
 * edges), by the same chain as the 1D blocks with b = max |x| over the
 * block's elements.  Both outputs keep the 1D layouts: the block's scale is
 * written for each of its rows in s_row[M][ceil(K/16)] and for each of its
 * columns in s_col[K][ceil(M/16)], and every element is coded with its
 * block's multiplier in q_row and in the transposed q_col. */
int orc_nvfp4_quantize_transpose_2d(const uint16_t *x, int64_t M, int64_t K, unsigned axis,
                                    float tensor_amax, uint8_t *q_row, uint8_t *s_row,
                                    uint8_t *q_col, uint8_t *s_col, float *sg_out)
{
    if (M <= 0 || K <= 0)
        return ORC_ERR_SHAPE;
    if (axis & ~3u)
        return ORC_ERR_ENUM;
    init_tables();
    float A = tensor_amax < 0.0f ? orc_absmax(x, M * K) : tensor_amax;
    float Sg = orc_nvfp4_global_scale(A);
    if (sg_out)
        *sg_out = Sg;
    if (!isfinite(A)) {
        nvfp4_nonfinite(M, K, axis, q_row, s_row, q_col, s_col);
        return ORC_OK;
    }
    const int64_t nbk = cdiv(K, 16), nbm = cdiv(M, 16), lk = cdiv(K, 2), lm = cdiv(M, 2);
#pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nbm; bi++) {
        double v[256];
        uint8_t c[256];
        const int nr = (int)(M - 16 * bi < 16 ? M - 16 * bi : 16);
        for (int64_t bj = 0; bj < nbk; bj++) {
            const int nc = (int)(K - 16 * bj < 16 ? K - 16 * bj : 16);
            for (int r = 0; r < nr; r++)
                for (int q = 0; q < nc; q++)
                    v[nc * r + q] = orc_bf16_value(x[(16 * bi + r) * K + 16 * bj + q]);
            uint8_t sb;
            nvfp4_block(v, nr * nc, Sg, c, 1, &sb);    /* codes in row-major order */
            for (int r = 0; r < nr && (axis & 1u); r++) {
                const int64_t m = 16 * bi + r;
                s_row[m * nbk + bj] = sb;
                pack_codes(c + nc * r, nc, 1, q_row + m * lk + 8 * bj);
            }
            for (int q = 0; q < nc && (axis & 2u); q++) {
                const int64_t k = 16 * bj + q;
                s_col[k * nbm + bi] = sb;
                pack_codes(c + q, nr, nc, q_col + k * lm + 8 * bi);
            }
        }
    }
    return ORC_OK;
}

/* Grouped NVFP4 (R10): G tensors stacked along rows, each quantised with its
 * own tensor amax and global scale (amax[g] when amax is given, else the
 * group's own max |x|), 1D or 2D scaling; outputs concatenated group after
 * group: q_row[M][ceil(K/2)] and s_row[M][ceil(K/16)] as for the stacked
 * rows; q_col / s_col group g's [K][ceil(rows/2)] / [K][ceil(rows/16)], one
 * group after the other; sg_out[g] (1 for an empty group, which owns no
 * output). */
int orc_nvfp4_quantize_transpose_grouped(const uint16_t *x, int64_t K, const int64_t *rows, int G,
                                         const float *amax, int two_d, unsigned axis,
                                         uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                         uint8_t *s_col, float *sg_out)
{
    if (G <= 0 || K <= 0)
        return ORC_ERR_SHAPE;
    int64_t r = 0, qc = 0, sc = 0;
    for (int g = 0; g < G; g++) {
        const int64_t m = rows[g];
        if (m < 0)
            return ORC_ERR_SHAPE;
        if (m == 0) {
            if (sg_out)
                sg_out[g] = 1.0f;
            continue;
        }
        const float A = amax ? amax[g] : -1.0f;
        int rc = (two_d ? orc_nvfp4_quantize_transpose_2d : orc_nvfp4_quantize_transpose)(
            x + r * K, m, K, axis, A, q_row ? q_row + r * cdiv(K, 2) : NULL,
            s_row ? s_row + r * cdiv(K, 16) : NULL, q_col ? q_col + qc : NULL,
            s_col ? s_col + sc : NULL, sg_out ? sg_out + g : NULL);
        if (rc != ORC_OK)
            return rc;
        r += m;
        qc += K * cdiv(m, 2);
        sc += K * cdiv(m, 16);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Array helpers for the self-tests (elementwise, no method arithmetic).     */
/* ------------------------------------------------------------------------ */

void orc_e4m3_encode_array(const double *v, uint8_t *out, int64_t n)
{
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_e4m3_encode(v[i]);
}

void orc_e5m2_encode_array(const double *v, uint8_t *out, int64_t n)
{
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_e5m2_encode(v[i]);
}

void orc_e2m1_encode_array(const double *v, uint8_t *out, int64_t n)
{
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_e2m1_encode(v[i]);
}

void orc_bf16_round_array(const double *v, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_round(v[i]);
}

/* which: 0 exp32, 1 gelu32, 2 dgelu32, 3 silu32, 4 dsilu32 */
void orc_unary32_array(int which, const float *v, float *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float a = v[i];
        out[i] = which == 0 ? orc_exp32(a) : which == 1 ? orc_gelu32(a)
               : which == 2 ? orc_dgelu32(a) : which == 3 ? orc_silu32(a) : orc_dsilu32(a);
    }
}

/* ------------------------------------------------------------------------ */
/* Bulk comparisons for the device qualification tests.  The GPU runs one of */
/* the library's per-element routines on every fp32 bit pattern of a range  */
/* (input i is the pattern first + i); these count the results that differ  */
/* from the rules above and report the first differing index (-1 if none).  */
/* The threads only split the range; the count and the minimum index do not  */
/* depend on how.                                                            */
/* ------------------------------------------------------------------------ */

static float f32_of_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* got[i]: bf16 bits of input i rounded to nearest even (NaN: any NaN). */
int64_t orc_check_bf16_round(const uint16_t *got, uint64_t first, int64_t n, int64_t *first_bad)
{
    int64_t bad = 0, fb = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : fb)
    for (int64_t i = 0; i < n; i++) {
        const float f = f32_of_bits((uint32_t)(first + (uint64_t)i));
        const uint16_t g = got[i];
        const int ok = isnan(f) ? ((g & 0x7F80) == 0x7F80 && (g & 0x7F) != 0)
                                : g == orc_bf16_round((double)f);
        if (!ok) {
            bad++;
            if (i < fb)
                fb = i;
        }
    }
    *first_bad = bad ? fb : -1;
    return bad;
}

/* got[j]: E2M1 codes of inputs 2j (low nibble) and 2j + 1 (high nibble);
 * NaN inputs are not compared. */
int64_t orc_check_e2m1(const uint8_t *got, uint64_t first, int64_t n, int64_t *first_bad)
{
    init_tables();
    int64_t bad = 0, fb = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : fb)
    for (int64_t i = 0; i < n; i++) {
        const float f = f32_of_bits((uint32_t)(first + (uint64_t)i));
        if (isnan(f))
            continue;
        const uint8_t g = (uint8_t)((got[i >> 1] >> (4 * (i & 1))) & 0xF);
        if (g != orc_e2m1_encode((double)f)) {
            bad++;
            if (i < fb)
                fb = i;
        }
    }
    *first_bad = bad ? fb : -1;
    return bad;
}

/* got[i]: saturating E4M3 code of input i; NaN inputs are not compared. */
int64_t orc_check_e4m3(const uint8_t *got, uint64_t first, int64_t n, int64_t *first_bad)
{
    init_tables();
    int64_t bad = 0, fb = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : fb)
    for (int64_t i = 0; i < n; i++) {
        const float f = f32_of_bits((uint32_t)(first + (uint64_t)i));
        if (isnan(f))
            continue;
        if (got[i] != orc_e4m3_encode((double)f)) {
            bad++;
            if (i < fb)
                fb = i;
        }
    }
    *first_bad = bad ? fb : -1;
    return bad;
}

/* got[i]: fp32 bits of e^x for input i (NaN: any NaN). */
int64_t orc_check_exp32(const uint32_t *got, uint64_t first, int64_t n, int64_t *first_bad)
{
    int64_t bad = 0, fb = INT64_MAX;
#pragma omp parallel for schedule(static) reduction(+ : bad) reduction(min : fb)
    for (int64_t i = 0; i < n; i++) {
        const float f = f32_of_bits((uint32_t)(first + (uint64_t)i));
        const float e = orc_exp32(f);
        uint32_t want;
        memcpy(&want, &e, 4);
        const int ok = isnan(f) ? isnan(f32_of_bits(got[i])) : got[i] == want;
        if (!ok) {
            bad++;
            if (i < fb)
                fb = i;
        }
    }
    *first_bad = bad ? fb : -1;
    return bad;
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
