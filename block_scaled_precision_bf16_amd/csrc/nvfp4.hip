// nvfp4.hip -- NVFP4 quantize-transpose for gfx950, plus the tensor absmax
// pass its global scale needs.  The pages time NVFP4 quantize-transpose
// kernels ("NVFP4 2D quantize-transpose kernel" table of TransformerEngine
// PR 3291, and its 1D bf16 kernel listed under "Patched but not
// measurable"); this is the 1D form: 16-element blocks along K for the
// row-wise output and along M for the transposed output.
//
// Same work layout as the MXFP8 cast: a lane owns 16 rows x 8 columns of a
// 128 x 256 workgroup tile, which makes each lane's 16 rows exactly one
// column block of the transposed output (no cross-lane work for dim1); a row
// block of 16 spans two lanes, combined with one DPP permute.
//
// Per block the scale chain costs three IEEE fp32 divisions (b/6, /S_g and
// the reciprocal); each element then costs one multiply and half of a packed
// hardware E2M1 convert.

#include "device_math.h"
#include "launch.h"

namespace mxk {

// Block scale byte and the element multiplier of one NVFP4 block whose
// largest magnitude has bf16 pattern `mag`.
__device__ __forceinline__ void nv_block(uint32_t mag, float sg, uint32_t &sbyte, float &inv)
{
    const float b = f32_bits(mag << 16);
    const float b6 = b / 6.0f;
    const float sq = b6 / sg;
    sbyte = e4m3_rne_sat(sq);
    const float den = e4m3_value(sbyte) * sg;
    inv = den == 0.0f ? 0.0f : 1.0f / den;
}

// Eight bf16 (four words) times inv -> eight E2M1 nibbles, element i in bits
// 4i..4i+3 (so element 2j is the low nibble of byte j).  A block whose
// multiplier overflowed to Inf (tensor scale below ~2^-120) takes the software
// encoder, which maps 0 * Inf to +0.
__device__ __forceinline__ uint32_t encode8_fp4(const uint32_t (&w)[4], float inv)
{
    if (__builtin_isinf(inv)) {
        uint32_t o = 0;
#pragma unroll
        for (int d = 0; d < 4; d++) {
            o |= e2m1_rne_sat(bf16_lo(w[d]) * inv) << (8 * d);
            o |= e2m1_rne_sat(bf16_hi(w[d]) * inv) << (8 * d + 4);
        }
        return o;
    }
    uint32_t o = e2m1x2<0>(bf16_lo(w[0]) * inv, bf16_hi(w[0]) * inv, 0u);
    o = e2m1x2<1>(bf16_lo(w[1]) * inv, bf16_hi(w[1]) * inv, o);
    o = e2m1x2<2>(bf16_lo(w[2]) * inv, bf16_hi(w[2]) * inv, o);
    return e2m1x2<3>(bf16_lo(w[3]) * inv, bf16_hi(w[3]) * inv, o);
}

// Rows 8q..8q+7 of one column (half HI of word d) times inv -> eight nibbles,
// row 8q+i in bits 4i..4i+3.
template <int HI>
__device__ __forceinline__ uint32_t encode8_fp4_col(const uint32_t (&w)[kRowsPerLane][4], int q,
                                                    int d, float inv)
{
    auto v = [&](int i) { return (HI ? bf16_hi(w[8 * q + i][d]) : bf16_lo(w[8 * q + i][d])) * inv; };
    if (__builtin_isinf(inv)) {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            o |= e2m1_rne_sat(v(i)) << (4 * i);
        return o;
    }
    uint32_t o = e2m1x2<0>(v(0), v(1), 0u);
    o = e2m1x2<1>(v(2), v(3), o);
    o = e2m1x2<2>(v(4), v(5), o);
    return e2m1x2<3>(v(6), v(7), o);
}

template <bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void nvfp4_kernel(Nv4Args a)
{
    const int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int tm = tile / a.tiles_k;
    const int tk = tile - tm * a.tiles_k;
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    const int half = lane >> 5, cl = lane & 31;
    const int64_t m0 = (int64_t)tm * kTileM + wave * (2 * kRowsPerLane) + half * kRowsPerLane;
    const int64_t k = (int64_t)tk * kTileK + cl * kColsPerLane;

    const float A = *a.amax;
    const float sg = A == 0.0f ? 1.0f : A / 2688.0f;
    if (a.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *a.sg_out = sg;
    // M and K are multiples of 16: a lane's 16 rows, and the two lanes of a
    // row block, are valid or invalid together.
    if (m0 >= a.M || k >= a.K)
        return;

    uint32_t w[kRowsPerLane][4];
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a.x + (m0 + r) * a.K + k);
        w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
    }

    uint32_t cmax[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        uint32_t m[4];
#pragma unroll
        for (int d = 0; d < 4; d++) {
            m[d] = w[r][d] & 0x7FFF7FFFu;
            if constexpr (COL)
                cmax[d] = pk_max_u16(cmax[d], m[d]);
        }
        if constexpr (ROW) {
            const uint32_t t = pk_max_u16(pk_max_u16(m[0], m[1]), pk_max_u16(m[2], m[3]));
            const uint32_t lo = t & 0xFFFFu, hi = t >> 16;
            uint32_t mag = lo > hi ? lo : hi;
            mag = max_xor1(mag);
            uint32_t sb;
            float inv;
            nv_block(mag, sg, sb, inv);
            const int64_t row = m0 + r;
            *reinterpret_cast<uint32_t *>(a.q_row + row * (a.K >> 1) + (k >> 1)) =
                encode8_fp4(w[r], inv);
            if ((lane & 1) == 0)
                a.s_row[row * (a.K >> 4) + (k >> 4)] = (uint8_t)sb;
        }
    }

    if constexpr (COL) {
#pragma unroll
        for (int c = 0; c < kColsPerLane; c++) {
            const int d = c >> 1, hi = c & 1;
            const uint32_t mag = hi ? (cmax[d] >> 16) : (cmax[d] & 0xFFFFu);
            uint32_t sb;
            float inv;
            nv_block(mag, sg, sb, inv);
            uint32_t o[2];
#pragma unroll
            for (int q = 0; q < 2; q++)
                o[q] = hi ? encode8_fp4_col<1>(w, q, d, inv) : encode8_fp4_col<0>(w, q, d, inv);
            *reinterpret_cast<uint2 *>(a.q_col + (k + c) * (a.M >> 1) + (m0 >> 1)) =
                make_uint2(o[0], o[1]);
            a.s_col[(k + c) * (a.M >> 4) + (m0 >> 4)] = (uint8_t)sb;
        }
    }
}

// ---------------------------------------------------------------------------
// Tensor absmax: largest |bf16| as the fp32 bit pattern (ordered like an
// unsigned integer for non-negative values), combined with atomic max.
// ---------------------------------------------------------------------------
__global__ void absmax_clear_kernel(uint32_t *amax_bits) { *amax_bits = 0u; }

__global__ __launch_bounds__(256) void absmax_kernel(const uint16_t *x, int64_t n,
                                                     uint32_t *amax_bits)
{
    const int64_t nvec = n >> 3;
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
        const uint4 v = reinterpret_cast<const uint4 *>(x)[i];
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                                     pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu)));
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
        const uint32_t t = x[(nvec << 3) + threadIdx.x] & 0x7FFFu;
        m = pk_max_u16(m, t);
    }
    uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    uint32_t mag = lo > hi ? lo : hi;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mag, off, 64);
        mag = mag > o ? mag : o;
    }
    if ((threadIdx.x & 63) == 0)
        atomicMax(amax_bits, mag << 16);
}

hipError_t launch_absmax(const uint16_t *x, int64_t n, float *amax, hipStream_t s)
{
    uint32_t *bits = reinterpret_cast<uint32_t *>(amax);
    hipLaunchKernelGGL(absmax_clear_kernel, dim3(1), dim3(1), 0, s, bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    int64_t blocks = ((n >> 3) + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, bits);
    return hipGetLastError();
}

template <bool ROW, bool COL>
static hipError_t launch_nv(const Nv4Args &a, hipStream_t s)
{
    hipLaunchKernelGGL((nvfp4_kernel<ROW, COL>), dim3(a.tiles_m * a.tiles_k), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_nvfp4(unsigned axis, const Nv4Args &a, hipStream_t s)
{
    switch (axis) {
    case 1u: return launch_nv<true, false>(a, s);
    case 2u: return launch_nv<false, true>(a, s);
    case 3u: return launch_nv<true, true>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mxk
