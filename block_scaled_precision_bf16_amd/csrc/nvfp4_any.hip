// nvfp4_any.hip -- NVFP4 quantize-transpose for shapes the tiled kernel
// (nvfp4.hip) does not take: any M and K, one tensor or groups stacked along
// M with any row counts.  Same arithmetic, bit for bit, 1D (16-element) or
// 2D (16 x 16) blocks; a block at the end of a line (2D: at the right or
// bottom edge) is quantised from the elements it has, and a line of n codes
// packs into ceil(n/2) bytes, the high nibble of an odd line's last byte 0.
// The pages time NVFP4 quantize-transpose kernels (TransformerEngine PR 3291
// page: table "NVFP4 2D quantize-transpose kernel" and the 1D bf16 kernel
// under "Patched but not measurable").
//
// Work as in the MXFP8 cast of any shape (any_common.h): a workgroup walks a
// 128-column strip in steps of 64 rows; thread t loads column t % 128 of 32
// rows, which are two 16-row column blocks of its own; four lanes of one wave
// take a row's 128 columns (eight 16-column blocks) from LDS for the
// row-wise output.  With 2D blocks the 16 lanes of a block reduce their
// column maxima with lane exchanges and the block scales reach the row pass
// through LDS.  A step's codes are 64 bytes per row and 32 bytes per
// transposed row.

#include "any_common.h"
#include "nv_block.h"

namespace mxk {

// LDS of one workgroup (32.3 KB: four workgroups per CU).
struct alignas(16) NvAnyStage {
    // bf16 values of the step (272-byte rows); once the row pass has read
    // row r, the first 64 bytes of that row hold row r's codes (the row's
    // four threads are lanes of one wave, whose reads precede its writes)
    uint16_t y[kAnyTileM][kAnyTileK + 8];
    // transposed codes, two steps per transposed row: step s at bytes
    // 32 (s % 2) .. 32 (s % 2) + 31 (80-byte rows)
    uint8_t qt[kAnyTileK][kAnyTileM + 16];
    uint8_t sc[kAnyTileK][4 * kAnyMaxWalk];   // column-block scales of the walk
    uint8_t blk[4][kAnyTileK / 16];           // 2D: the step's 16 x 16 block scales
    float inv[128];                           // multiplier of each scale byte
};

struct NvAnyView {
    const uint16_t *x;
    int64_t M;
    uint8_t *q_row, *s_row, *q_col, *s_col;
};

// Largest 15-bit magnitude of 16 elements (8 packed words).
__device__ __forceinline__ uint32_t max16(const uint32_t *w)
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        m = pk_max_u16(m, w[i] & 0x7FFF7FFFu);
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    return lo > hi ? lo : hi;
}

// Sixteen codes (8 packed words of elements) with multiplier inv -> 8 bytes;
// all zero for a tensor whose amax is not finite.
__device__ __forceinline__ uint2 nv_codes16(const uint32_t *w, float inv, bool nonfin)
{
    const uint32_t a[4] = {w[0], w[1], w[2], w[3]}, b[4] = {w[4], w[5], w[6], w[7]};
    const uint2 o = make_uint2(encode8_fp4(a, inv), encode8_fp4(b, inv));
    return nonfin ? make_uint2(0u, 0u) : o;
}

// One 64 x 128 step (the s-th of the walk) at rows m0, columns k0; w: this
// thread's column (column k0 + t % 128, rows m0 + 32 (t / 128) + i).
template <bool TWO_D>
__device__ __forceinline__ void nv_any_step(const Nv4Args &a, const NvAnyView &v, NvAnyStage &st,
                                            const DivBy &sg, bool nonfin, const uint32_t (&w)[16],
                                            int64_t m0, int tk, int s, bool last_step,
                                            unsigned axis)
{
    const int t = (int)threadIdx.x;
    const int c = t & (kAnyTileK - 1);
    const int h = __builtin_amdgcn_readfirstlane(t >> 7);   // uniform per wave
    const int64_t k0 = (int64_t)tk * kAnyTileK;
    const bool row = axis & 1u, col = (axis & 2u) != 0;

    if (row) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            st.y[32 * h + 2 * i][c] = (uint16_t)(w[i] & 0xFFFFu);
            st.y[32 * h + 2 * i + 1][c] = (uint16_t)(w[i] >> 16);
        }
    }
    if (col || TWO_D) {
        uint2 q[2];
#pragma unroll
        for (int bq = 0; bq < 2; bq++) {                  // rows 32 h + 16 bq .. + 15
            uint32_t mag = max16(&w[8 * bq]);
            if constexpr (TWO_D) {
                // the 16 x 16 block: this column and the 15 beside it (16
                // consecutive lanes of the wave)
#pragma unroll
                for (int d = 1; d < 16; d <<= 1) {
                    const uint32_t o = (uint32_t)__shfl_xor((int)mag, d, 64);
                    mag = mag > o ? mag : o;
                }
            }
            const uint32_t sb = nonfin ? 0x7Fu : nv_scale(mag, sg);
            if (TWO_D && (c & 15) == 0)
                st.blk[2 * h + bq][c >> 4] = (uint8_t)sb;
            q[bq] = nv_codes16(&w[8 * bq], st.inv[sb], nonfin);
            st.sc[c][4 * s + 2 * h + bq] = (uint8_t)sb;
        }
        if (col)
            *reinterpret_cast<uint4 *>(&st.qt[c][32 * (s & 1) + 16 * h]) =
                make_uint4(q[0].x, q[0].y, q[1].x, q[1].y);
    }
    __syncthreads();
    if (row) {
        const int r = t >> 2, qq = t & 3;                 // row r, columns 32 qq .. 32 qq + 31
        uint32_t wr[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint4 u = *reinterpret_cast<const uint4 *>(&st.y[r][32 * qq + 8 * j]);
            wr[4 * j] = u.x; wr[4 * j + 1] = u.y; wr[4 * j + 2] = u.z; wr[4 * j + 3] = u.w;
        }
        const int64_t nbk = (a.K + 15) >> 4;
        const rsrc_t rs = make_rsrc(v.s_row, m0 * nbk, v.M * nbk);
        uint2 o[2];
#pragma unroll
        for (int bq = 0; bq < 2; bq++) {
            const uint32_t sb = TWO_D ? (uint32_t)st.blk[r >> 4][2 * qq + bq]
                                      : (nonfin ? 0x7Fu : nv_scale(max16(&wr[8 * bq]), sg));
            o[bq] = nv_codes16(&wr[8 * bq], st.inv[sb], nonfin);
            const int64_t b = (int64_t)8 * tk + 2 * qq + bq;
            const bool ok = m0 + r < v.M && b < nbk;
            buf_store1(rs, ok ? (uint32_t)(r * nbk + b) : kDead, (uint8_t)sb);
        }
        uint8_t *qd = reinterpret_cast<uint8_t *>(st.y[r]) + 16 * qq;   // over row r's values, read
        *reinterpret_cast<uint4 *>(qd) = make_uint4(o[0].x, o[0].y, o[1].x, o[1].y);
    }
    __syncthreads();
    const int mrem = (int)(v.M - m0 < kAnyTileM ? v.M - m0 : kAnyTileM);
    if (row) {
        const int64_t lk = (a.K + 1) >> 1;                // bytes per row of q_row
        flush_rows<kAnyTileK / 2>(v.q_row, lk, m0, 64 * (int64_t)tk, v.M * lk, mrem,
                                  (int)(lk - 64 * tk < 64 ? lk - 64 * tk : 64),
                                  reinterpret_cast<const uint8_t *>(st.y[0]), (int)sizeof(st.y[0]));
    }
    if (col)
        flush_cols<kAnyTileM / 2>(v.q_col, (v.M + 1) >> 1, k0, a.K, m0 >> 1, (mrem + 1) >> 1, s,
                                  last_step, st.qt[0], (int)sizeof(st.qt[0]));
    __syncthreads();
}

// Column scales of a walk over steps t0 .. t0 + n - 1 (blocks 4 t0 ..
// 4 t0 + 4n - 1) of strip tk into s_col[K][ceil(M / 16)].
__device__ __forceinline__ void nv_any_flush_scol(const Nv4Args &a, const NvAnyView &v,
                                                  const NvAnyStage &st, int t0, int n, int tk)
{
    const int64_t k0 = (int64_t)tk * kAnyTileK;
    const int64_t nb = (v.M + 15) >> 4;
    const int64_t jb = 4 * (int64_t)t0;
    const rsrc_t rs = make_rsrc(v.s_col, k0 * nb + jb, a.K * nb);
    for (int idx = (int)threadIdx.x; idx < kAnyTileK * 4 * kAnyMaxWalk; idx += kThreads) {
        const int c = idx / (4 * kAnyMaxWalk), jj = idx % (4 * kAnyMaxWalk);
        const bool ok = jj < 4 * n && k0 + c < a.K && jb + jj < nb;
        buf_store1(rs, ok ? (uint32_t)(c * nb + jj) : kDead, st.sc[c][ok ? jj : 0]);
    }
}

// Walk w (numbered across groups) of strip tk; group g holds walks
// walk0[g] .. walk0[g + 1] - 1 of len[g] steps, its own amax (a.amax[g]) and
// global scale.  Workgroup 0 writes every group's global scale (1 for an
// empty group).
template <bool TWO_D>
__global__ __launch_bounds__(kThreads, 4) void nvfp4_any_kernel(Nv4Args a, GroupTable gt,
                                                                unsigned axis)
{
    __shared__ NvAnyStage st;
    const int t = (int)threadIdx.x;
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int walk = job / a.tiles_k;
    const int tk = job - walk * a.tiles_k;
    if (a.sg_out != nullptr && blockIdx.x == 0 && t < gt.count)
        a.sg_out[t] = gt.row0[t + 1] == gt.row0[t] ? 1.0f : nv_global_scale(a.amax[t]);
    int g = 0;
    while (g + 1 < gt.count && gt.walk0[g + 1] <= walk)
        g++;
    const int64_t r0 = gt.row0[g];
    NvAnyView v;
    v.M = gt.row0[g + 1] - r0;
    v.x = a.x + r0 * a.K;
    v.q_row = a.q_row ? a.q_row + r0 * ((a.K + 1) >> 1) : nullptr;
    v.s_row = a.s_row ? a.s_row + r0 * ((a.K + 15) >> 4) : nullptr;
    v.q_col = a.q_col ? a.q_col + gt.qcol_off[g] : nullptr;
    v.s_col = a.s_col ? a.s_col + gt.scol_off[g] : nullptr;

    const float sgf = nv_global_scale(a.amax[g]);
    const bool nonfin = !__builtin_isfinite(sgf);   // an Inf or NaN in the tensor
    const DivBy sg = div_by_prepare(nonfin ? 1.0f : sgf);
    if (t < 128)
        st.inv[t] = nv_inverse((uint32_t)t, sgf);
    __syncthreads();

    const int len = gt.len[g];
    const int t0 = (walk - gt.walk0[g]) * len;
    const int tiles_m = (int)((v.M + kAnyTileM - 1) / kAnyTileM);
    const int n = tiles_m - t0 < len ? tiles_m - t0 : len;
    const int h = __builtin_amdgcn_readfirstlane(t >> 7);
    const int64_t k = (int64_t)tk * kAnyTileK + (t & (kAnyTileK - 1));
    for (int s = 0; s < n; s++) {
        uint32_t w[16];
        load_column32(v.x, a.K, v.M, (int64_t)(t0 + s) * kAnyTileM + 32 * h, k, k < a.K, w);
        nv_any_step<TWO_D>(a, v, st, sg, nonfin, w, (int64_t)(t0 + s) * kAnyTileM, tk, s, s + 1 == n,
                           axis);
    }
    if (axis & 2u)
        nv_any_flush_scol(a, v, st, t0, n, tk);
}

hipError_t launch_nvfp4_any(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                            hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)gt.walk0[gt.count] * a.tiles_k));
    if (two_d)
        hipLaunchKernelGGL(nvfp4_any_kernel<true>, grid, dim3(kThreads), 0, s, a, gt, axis);
    else
        hipLaunchKernelGGL(nvfp4_any_kernel<false>, grid, dim3(kThreads), 0, s, a, gt, axis);
    return hipGetLastError();
}

}  // namespace mxk
