// mx_cast.hip -- MXFP8 cast kernels for gfx950: row-wise (dim0), column-wise
// (dim1, transposed output) or both in one pass over the bf16 input,
// optionally with a fused GELU / dGELU / SwiGLU / GeGLU pre-op and a dbias
// column sum.  These are the kernels the TransformerEngine PR 3291 page
// times ("MXFP8 generic quantize kernel", "MXFP8 specialized cast-only kernel
// (bidimensional)", "MXFP8 gated (swiglu / geglu) kernel") and the torchao
// dim1 cast of PR 12, designed here for CDNA4.
//
// Layout of the work: a workgroup (4 waves) owns a 128-row x 256-column
// tile.  A lane owns 16 consecutive rows x 8 consecutive columns, loaded as
// 16 128-bit loads; lanes 0-31 of a wave hold rows 0-15 and lanes 32-63 rows
// 16-31 of the same 256 columns, so each wave load instruction reads two
// 512-byte row segments (fully coalesced) and a wave covers exactly one
// 32-row column block.  The column-wise (dim1) amax of a column is the max of
// two lanes' in-register maxima (one exchange between lane l and l^32), and
// each lane then converts and stores its own 16 bytes of the transposed row,
// so the dim1 path needs no transpose through LDS.  The row-wise amax spans 4
// lanes (4 x 8 = 32 columns), reduced with two DPP quad permutes.  Row
// outputs leave as 8-byte stores (256 contiguous bytes per half-wave);
// column outputs as 16-byte stores, the 8 lane-halves of a workgroup
// completing each 128-byte line of the transposed tensor.  LDS is used only
// for the dbias cross-wave sum, as a statically declared array (its address
// never passes through an integer: the fix the PR 3291 page is about).
//
// Every element costs one multiply by the exact power-of-two inverse of its
// block scale (the torchao PR 12 page: divisions per element made the dim1
// cast compute bound) and an integer round-to-nearest-even E4M3 encode.

#include "device_math.h"
#include "launch.h"

namespace mxk {

__device__ __forceinline__ float half_value(uint32_t w, int hi)
{
    return hi ? bf16_hi(w) : bf16_lo(w);
}

// Four bf16 (two packed words) times inv -> four E4M3 bytes in one word.
__device__ __forceinline__ uint32_t encode4(uint32_t w0, uint32_t w1, float inv)
{
    return e4m3_rne_sat(bf16_lo(w0) * inv) | (e4m3_rne_sat(bf16_hi(w0) * inv) << 8) |
           (e4m3_rne_sat(bf16_lo(w1) * inv) << 16) | (e4m3_rne_sat(bf16_hi(w1) * inv) << 24);
}

template <int OP>
__device__ __forceinline__ void load_rows(const MxArgs &a, int64_t m0, int64_t k, bool live,
                                          uint32_t (&w)[kRowsPerLane][4])
{
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        if (live) {
            const uint16_t *px = a.x + (m0 + r) * a.ldx + k;
            const uint4 v = *reinterpret_cast<const uint4 *>(px);
            if constexpr (OP == OP_PLAIN) {
                w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
            } else {
                uint4 b = v;   // GELU has no second operand
                if constexpr (OP != OP_GELU) {
                    const uint16_t *pb = (OP == OP_DGELU) ? a.aux + (m0 + r) * a.ldx + k
                                                          : px + a.lin_off;
                    b = *reinterpret_cast<const uint4 *>(pb);
                }
                w[r][0] = fused_pair<OP>(v.x, b.x);
                w[r][1] = fused_pair<OP>(v.y, b.y);
                w[r][2] = fused_pair<OP>(v.z, b.z);
                w[r][3] = fused_pair<OP>(v.w, b.w);
            }
        } else {
            w[r][0] = w[r][1] = w[r][2] = w[r][3] = 0u;
        }
    }
}

template <int OP, bool ROW, bool COL, bool DBIAS>
__global__ __launch_bounds__(kThreads) void mx_cast_kernel(MxArgs a)
{
    const int tile = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int tm = tile / a.tiles_k;
    const int tk = tile - tm * a.tiles_k;
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    const int half = lane >> 5, cl = lane & 31;
    const int64_t mb = (int64_t)tm * kTileM + wave * (2 * kRowsPerLane);  // column block
    const int64_t m0 = mb + half * kRowsPerLane;                            // first row
    const int64_t k = (int64_t)tk * kTileK + cl * kColsPerLane;
    const bool wave_live = mb < a.M;   // M is a multiple of 32: whole waves
    if (!DBIAS && !wave_live)
        return;
    const bool live = wave_live && k < a.K;

    uint32_t w[kRowsPerLane][4];
    load_rows<OP>(a, m0, k, live, w);

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
            mag = max_xor2(mag);
            const uint32_t sb = e8m0_from_mag(mag);
            const float inv = e8m0_inverse(sb);
            uint2 o;
            o.x = encode4(w[r][0], w[r][1], inv);
            o.y = encode4(w[r][2], w[r][3], inv);
            if (sb == 0xFFu)
                o.x = o.y = 0x7F7F7F7Fu;
            if (live) {
                const int64_t row = m0 + r;
                *reinterpret_cast<uint2 *>(a.q_row + row * a.K + k) = o;
                if ((lane & 3) == 0)
                    a.s_row[row * (a.K >> 5) + (k >> 5)] = (uint8_t)sb;
            }
        }
    }

    if constexpr (COL) {
        // the other 16 rows of each column block are in lane l ^ 32
#pragma unroll
        for (int d = 0; d < 4; d++)
            cmax[d] = pk_max_u16(cmax[d], (uint32_t)__shfl_xor((int)cmax[d], 32, 64));
#pragma unroll
        for (int c = 0; c < kColsPerLane; c++) {
            const int d = c >> 1, hi = c & 1;
            const uint32_t mag = hi ? (cmax[d] >> 16) : (cmax[d] & 0xFFFFu);
            const uint32_t sb = e8m0_from_mag(mag);
            const float inv = e8m0_inverse(sb);
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                o[j] = e4m3_rne_sat(half_value(w[4 * j + 0][d], hi) * inv) |
                       (e4m3_rne_sat(half_value(w[4 * j + 1][d], hi) * inv) << 8) |
                       (e4m3_rne_sat(half_value(w[4 * j + 2][d], hi) * inv) << 16) |
                       (e4m3_rne_sat(half_value(w[4 * j + 3][d], hi) * inv) << 24);
                if (sb == 0xFFu)
                    o[j] = 0x7F7F7F7Fu;
            }
            if (live) {
                *reinterpret_cast<uint4 *>(a.q_col + (k + c) * a.M + m0) =
                    make_uint4(o[0], o[1], o[2], o[3]);
                if (half == 0)
                    a.s_col[(k + c) * (a.M >> 5) + (mb >> 5)] = (uint8_t)sb;
            }
        }
    }

    if constexpr (DBIAS) {
        // Column sums of y: over this lane's 16 rows in order, then over the 8
        // lane-halves of the workgroup in order; one fp32 partial per
        // (tile row, column).
        __shared__ float4 red[2 * kWaves][kTileK / 4];
        float s[kColsPerLane];
#pragma unroll
        for (int c = 0; c < kColsPerLane; c++) {
            float acc = 0.0f;
#pragma unroll
            for (int r = 0; r < kRowsPerLane; r++)
                acc += half_value(w[r][c >> 1], c & 1);
            s[c] = acc;
        }
        const int slot = 2 * wave + half;
        red[slot][cl * 2] = make_float4(s[0], s[1], s[2], s[3]);
        red[slot][cl * 2 + 1] = make_float4(s[4], s[5], s[6], s[7]);
        __syncthreads();
        const int t = (int)threadIdx.x;   // one column of the tile per thread
        const int64_t kc = (int64_t)tk * kTileK + t;
        if (kc < a.K) {
            const float *flat = reinterpret_cast<const float *>(red);
            float acc = flat[t];
#pragma unroll
            for (int v = 1; v < 2 * kWaves; v++)
                acc += flat[v * kTileK + t];
            a.partials[(int64_t)tm * a.K + kc] = acc;
        }
    }
}

// dbias[k] = sum over tile rows t (in order) of partials[t][k].
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float *partials, int tiles_m,
                                                           int64_t K, float *dbias)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K)
        return;
    float acc = 0.0f;
    for (int t = 0; t < tiles_m; t++)
        acc += partials[(int64_t)t * K + k];
    dbias[k] = acc;
}

// y = fused value of each element; 8 elements per thread.  Gated ops read
// the row [gate | linear] of width 2K.
template <int OP>
__global__ __launch_bounds__(256) void fused_values_kernel(const uint16_t *x, const uint16_t *aux,
                                                           int64_t M, int64_t K, uint16_t *y)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= M * K)
        return;
    const int64_t row = i / K, col = i - row * K;
    const bool gated = OP == OP_SWIGLU || OP == OP_GEGLU;
    const uint16_t *pa = gated ? x + row * 2 * K + col : x + i;
    const uint16_t *pb = gated ? pa + K : aux + i;
    const uint4 va = *reinterpret_cast<const uint4 *>(pa);
    const uint4 vb = *reinterpret_cast<const uint4 *>(pb);
    uint4 o;
    o.x = fused_pair<OP>(va.x, vb.x);
    o.y = fused_pair<OP>(va.y, vb.y);
    o.z = fused_pair<OP>(va.z, vb.z);
    o.w = fused_pair<OP>(va.w, vb.w);
    *reinterpret_cast<uint4 *>(y + i) = o;
}

template <int OP, bool ROW, bool COL, bool DBIAS>
static hipError_t launch_one(const MxArgs &a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_k;
    hipLaunchKernelGGL((mx_cast_kernel<OP, ROW, COL, DBIAS>), dim3(blocks), dim3(kThreads), 0,
                       s, a);
    return hipGetLastError();
}

template <int OP, bool DBIAS>
static hipError_t launch_axis(unsigned axis, const MxArgs &a, hipStream_t s)
{
    switch (axis) {
    case 1u: return launch_one<OP, true, false, DBIAS>(a, s);
    case 2u: return launch_one<OP, false, true, DBIAS>(a, s);
    case 3u: return launch_one<OP, true, true, DBIAS>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mx_cast(int op, unsigned axis, bool dbias, const MxArgs &a, hipStream_t s)
{
    switch (op) {
    case OP_PLAIN:
        return dbias ? launch_axis<OP_PLAIN, true>(axis, a, s) : launch_axis<OP_PLAIN, false>(axis, a, s);
    case OP_GELU:
        return dbias ? launch_axis<OP_GELU, true>(axis, a, s) : launch_axis<OP_GELU, false>(axis, a, s);
    case OP_DGELU:
        return dbias ? launch_axis<OP_DGELU, true>(axis, a, s) : launch_axis<OP_DGELU, false>(axis, a, s);
    case OP_SWIGLU:
        return launch_axis<OP_SWIGLU, false>(axis, a, s);
    case OP_GEGLU:
        return launch_axis<OP_GEGLU, false>(axis, a, s);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_dbias_reduce(const float *partials, int tiles_m, int64_t K, float *dbias,
                               hipStream_t s)
{
    const int64_t blocks = (K + 255) / 256;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials,
                       tiles_m, K, dbias);
    return hipGetLastError();
}

hipError_t launch_fused_values(int op, const uint16_t *x, const uint16_t *aux, int64_t M,
                               int64_t K, uint16_t *y, hipStream_t s)
{
    const int64_t threads = M * K / 8;
    const dim3 grid((unsigned)((threads + 255) / 256));
    switch (op) {
    case OP_GELU:
        hipLaunchKernelGGL(fused_values_kernel<OP_GELU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    case OP_DGELU:
        hipLaunchKernelGGL(fused_values_kernel<OP_DGELU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    case OP_SWIGLU:
        hipLaunchKernelGGL(fused_values_kernel<OP_SWIGLU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    case OP_GEGLU:
        hipLaunchKernelGGL(fused_values_kernel<OP_GEGLU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mxk
