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
// Every element costs a packed integer clamp and half of a packed scaled
// convert that applies the block's power-of-two scale exactly (the torchao
// PR 12 page: divisions per element made the dim1 cast compute bound; here
// there is not even a multiply per element).

#include "device_math.h"
#include "launch.h"

namespace mxk {

__device__ __forceinline__ float half_value(uint32_t w, int hi)
{
    return hi ? bf16_hi(w) : bf16_lo(w);
}

// Row r's 8 elements (4 words w, magnitudes mag) with scale byte b -> 8 E4M3
// bytes.
__device__ __forceinline__ uint2 encode8_row(const uint32_t (&w)[4], const uint32_t (&mag)[4],
                                             uint32_t b)
{
    const uint32_t lim = sat_limit2(b);
    const float sc = e8m0_operand(b);
    uint2 o;
    o.x = e4m3x2_scaled<false>(clamp_pair(w[0], mag[0], lim), sc, 0u);
    o.x = e4m3x2_scaled<true>(clamp_pair(w[1], mag[1], lim), sc, o.x);
    o.y = e4m3x2_scaled<false>(clamp_pair(w[2], mag[2], lim), sc, 0u);
    o.y = e4m3x2_scaled<true>(clamp_pair(w[3], mag[3], lim), sc, o.y);
    return o;
}

// Rows 2i and 2i+1 of one column (half HI of word d) as a packed bf16 pair.
template <int HI>
__device__ __forceinline__ uint32_t col_pair(const uint32_t (&w)[kRowsPerLane][4], int i, int d)
{
    return __builtin_amdgcn_perm(w[2 * i + 1][d], w[2 * i][d], HI ? 0x07060302u : 0x05040100u);
}

// One column's 16 rows (half HI of word d) with scale byte b -> 16 E4M3 bytes,
// row 0 in the lowest byte.
template <int HI>
__device__ __forceinline__ uint4 encode16_col(const uint32_t (&w)[kRowsPerLane][4], int d,
                                              uint32_t b)
{
    const uint32_t lim = sat_limit2(b);
    const float sc = e8m0_operand(b);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t p0 = col_pair<HI>(w, 2 * j, d), p1 = col_pair<HI>(w, 2 * j + 1, d);
        const uint32_t t = e4m3x2_scaled<false>(clamp_pair(p0, p0 & 0x7FFF7FFFu, lim), sc, 0u);
        o[j] = e4m3x2_scaled<true>(clamp_pair(p1, p1 & 0x7FFF7FFFu, lim), sc, t);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int OP>
__device__ __forceinline__ void load_rows(const MxArgs &a, const uint16_t *px,
                                          const uint16_t *pg, uint32_t (&w)[kRowsPerLane][4])
{
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(px);
        if constexpr (OP == OP_PLAIN) {
            w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        } else {
            uint4 b = v;   // GELU has no second operand
            if constexpr (OP == OP_DGELU)
                b = *reinterpret_cast<const uint4 *>(pg);
            else if constexpr (OP == OP_SWIGLU || OP == OP_GEGLU)
                b = *reinterpret_cast<const uint4 *>(px + a.lin_off);
            w[r][0] = fused_pair<OP>(v.x, b.x);
            w[r][1] = fused_pair<OP>(v.y, b.y);
            w[r][2] = fused_pair<OP>(v.z, b.z);
            w[r][3] = fused_pair<OP>(v.w, b.w);
            // one row's activation math at a time: interleaving rows only
            // multiplies the live temporaries
            __builtin_amdgcn_sched_barrier(0);
        }
        px += a.ldx;
        pg += a.ldx;
    }
}

// Row-wise blocks of this lane's 16 rows: amax over 4 lanes x 8 columns,
// scale, convert, store.  Column maxima are accumulated on the way.
template <bool ROW, bool COL>
__device__ __forceinline__ void row_pass(const MxArgs &a, const uint32_t (&w)[kRowsPerLane][4],
                                         int64_t m0, int64_t k, int lane, uint8_t *srow,
                                         uint32_t (&cmax)[4])
{
    uint8_t *qr = a.q_row + m0 * a.K + k;
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
            uint2 o = encode8_row(w[r], m, sb);
            if (sb == 0xFFu)
                o.x = o.y = 0x7F7F7F7Fu;
            *reinterpret_cast<uint2 *>(qr) = o;
            if ((lane & 3) == 0)
                srow[r * (kTileK / 32)] = (uint8_t)sb;
            qr += a.K;
        }
    }
}

// LDS staging of the column-wise output.  q: one sub-tile's transposed E4M3
// tile, q_col rows k0..k0+255, 128 bytes each (sub-tile rows m..m+127), as 8
// chunks of 16 bytes; chunk j of row kl is stored at chunk position
// j ^ ((kl >> 3) & 7): the 32 lanes of a half-wave write rows 8 apart (one
// per lane), the 8 threads that read a row back read its 8 chunks, and both
// patterns then cover all banks.  s: the column-block scales of the whole
// strip segment the workgroup walks (4 per sub-tile), written out once.
struct ColStage {
    uint4 q[kTileK][kTileM / 16];            // 32 KB
    uint8_t s[kTileK][4 * kMaxGroup];        // 16 KB
};

__device__ __forceinline__ int stage_chunk(int kl, int j) { return j ^ ((kl >> 3) & 7); }

// Column-wise blocks of sub-tile g: the 32 rows of a column block are this
// lane's 16 and those of lane l ^ 32; each lane converts its own 16 bytes of
// each column and puts them into the staging tile.
__device__ __forceinline__ void col_pass(ColStage &st, const uint32_t (&w)[kRowsPerLane][4],
                                         int wave, int half, int cl, int g, uint32_t (&cmax)[4])
{
#pragma unroll
    for (int d = 0; d < 4; d++)
        cmax[d] = pk_max_u16(cmax[d], (uint32_t)__shfl_xor((int)cmax[d], 32, 64));
#pragma unroll
    for (int c = 0; c < kColsPerLane; c++) {
        const int d = c >> 1, hi = c & 1;
        const uint32_t mag = hi ? (cmax[d] >> 16) : (cmax[d] & 0xFFFFu);
        const uint32_t sb = e8m0_from_mag(mag);
        uint4 o = hi ? encode16_col<1>(w, d, sb) : encode16_col<0>(w, d, sb);
        if (sb == 0xFFu)
            o = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
        const int kl = cl * kColsPerLane + c;
        st.q[kl][stage_chunk(kl, 2 * wave + half)] = o;
        if (half == 0)
            st.s[kl][4 * g + wave] = (uint8_t)sb;
    }
}

// Write the staged transposed tile of sub-tile tm: thread t writes 16-byte
// chunk t % 8 of q_col rows t / 8 + 32 i (i = 0..7), so each wave store
// instruction covers 8 whole 128-byte lines.
__device__ __forceinline__ void col_flush_q(const MxArgs &a, const ColStage &st, int tm, int tk)
{
    const int t = (int)threadIdx.x;
    const int jr = t & 7;
    const int64_t mt = (int64_t)tm * kTileM;
    const int64_t k0 = (int64_t)tk * kTileK;
    const bool chunk_live = mt + 16 * jr < a.M;   // M is a multiple of 32
#pragma unroll
    for (int i = 0; i < kTileK / 32; i++) {
        const int kr = (t >> 3) + 32 * i;
        if (chunk_live && k0 + kr < a.K)
            *reinterpret_cast<uint4 *>(a.q_col + (k0 + kr) * a.M + mt + 16 * jr) =
                st.q[kr][stage_chunk(kr, jr)];
    }
}

// Write the strip segment's column scales: thread t owns column k0 + t and
// writes its 4 n scale bytes (n sub-tiles) as 16-byte stores when the row of
// s_col allows it (a whole 64-byte chunk for a 16-deep walk), else bytewise.
__device__ __forceinline__ void col_flush_s(const MxArgs &a, const ColStage &st, int rg, int tk,
                                            int n)
{
    const int t = (int)threadIdx.x;
    const int64_t k0 = (int64_t)tk * kTileK;
    if (k0 + t >= a.K)
        return;
    const int64_t nblk = a.M >> 5;                        // scales per column
    const int64_t first = (int64_t)rg * a.group * 4;      // this segment's first block
    const int64_t left = nblk - first;
    const int count = (int)(left < 4 * n ? left : 4 * n);
    uint8_t *dst = a.s_col + (k0 + t) * nblk + first;
    if (((nblk | first) & 15) == 0 && (count & 15) == 0) {
        for (int i = 0; i < count; i += 16)
            *reinterpret_cast<uint4 *>(dst + i) = *reinterpret_cast<const uint4 *>(&st.s[t][i]);
    } else {
        for (int i = 0; i < count; i++)
            dst[i] = st.s[t][i];
    }
}

// Row scales of a sub-tile, staged as [128 rows][8 blocks] bytes: thread
// t < 128 writes row t's 8 scale bytes with one 8-byte store (instead of 8
// one-byte stores from 8 lanes).
__device__ __forceinline__ void srow_flush(const MxArgs &a, const uint8_t (&srow)[kTileM][kTileK / 32],
                                           int tm, int tk)
{
    const int t = (int)threadIdx.x;
    const int64_t row = (int64_t)tm * kTileM + t;
    if (t >= kTileM || row >= a.M)
        return;
    const int64_t k0 = (int64_t)tk * kTileK;
    uint8_t *dst = a.s_row + row * (a.K >> 5) + (k0 >> 5);
    const int64_t blocks = (a.K - k0) >> 5;   // scale bytes of this tile inside K
    if ((a.K & 255) == 0) {
        *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(srow[t]);
    } else {
#pragma unroll
        for (int b = 0; b < kTileK / 32; b++)
            if (b < blocks)
                dst[b] = srow[t][b];
    }
}

// Raw bf16 words of this lane's 16 rows of sub-tile tm (no pre-op).
__device__ __forceinline__ void load_plain(const MxArgs &a, int64_t m0, int64_t k,
                                           uint32_t (&w)[kRowsPerLane][4])
{
    const uint16_t *px = a.x + m0 * a.ldx + k;
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(px);
        w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        px += a.ldx;
    }
}

// One sub-tile of the walk: row pass (direct row stores, row scales to LDS),
// column pass into LDS, then the staged output leaves as whole lines.
template <bool ROW, bool COL, bool DBIAS>
__device__ __forceinline__ void tile_step(const MxArgs &a, const uint32_t (&w)[kRowsPerLane][4],
                                          uint8_t (&srow)[kTileM][kTileK / 32], ColStage *st,
                                          int tm, int tk, int g, float (&dsum)[kColsPerLane])
{
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int half = lane >> 5, cl = lane & 31;
    const int64_t mb = (int64_t)tm * kTileM + wave * (2 * kRowsPerLane);
    const int64_t m0 = mb + half * kRowsPerLane;
    const int64_t k = (int64_t)tk * kTileK + cl * kColsPerLane;
    // M is a multiple of 32, so a wave is wholly inside or outside; a column
    // group of 8 is wholly inside or outside K, and so are the 4-lane row
    // blocks and the l / l^32 pairs that exchange data.
    const bool live = mb < a.M && k < a.K;
    if (live) {
        uint32_t cmax[4] = {0u, 0u, 0u, 0u};
        row_pass<ROW, COL>(a, w, m0, k, lane, &srow[wave * 32 + half * 16][cl >> 2], cmax);
        if constexpr (COL)
            col_pass(*st, w, wave, half, cl, g, cmax);
        if constexpr (DBIAS) {
#pragma unroll
            for (int c = 0; c < kColsPerLane; c++) {
                float acc = dsum[c];
#pragma unroll
                for (int r = 0; r < kRowsPerLane; r++)
                    acc += half_value(w[r][c >> 1], c & 1);
                dsum[c] = acc;
            }
        }
    }
    __syncthreads();
    if constexpr (COL)
        col_flush_q(a, *st, tm, tk);
    if constexpr (ROW)
        srow_flush(a, srow, tm, tk);
    __syncthreads();   // the staging buffers are reused by the next sub-tile
}

// A workgroup walks a strip of 256 columns down `group` sub-tiles of 128 rows.
// Walking keeps the strip's column scales together (so they leave as whole
// 64-byte chunks rather than 4-byte pieces) and, for the plain cast, lets the
// next sub-tile's loads overlap the current sub-tile's conversion.
template <int OP, bool ROW, bool COL, bool DBIAS>
__global__ __launch_bounds__(kThreads) void mx_cast_kernel(MxArgs a)
{
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int rg = job / a.tiles_k;
    const int tk = job - rg * a.tiles_k;
    const int tm0 = rg * a.group;
    const int n = (a.tiles_m - tm0) < a.group ? (a.tiles_m - tm0) : a.group;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    const int half = lane >> 5, cl = lane & 31;
    const int64_t k = (int64_t)tk * kTileK + cl * kColsPerLane;
    const int64_t row_off = wave * (2 * kRowsPerLane) + half * kRowsPerLane;

    __shared__ __align__(16) uint8_t srow[kTileM][kTileK / 32];
    ColStage *st = nullptr;
    if constexpr (COL) {
        __shared__ ColStage stage;
        st = &stage;
    }
    float dsum[kColsPerLane] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto live = [&](int g) { return (int64_t)(tm0 + g) * kTileM + wave * 32 < a.M && k < a.K; };

    if constexpr (OP == OP_PLAIN) {
        // software pipeline over two register sets
        uint32_t wa[kRowsPerLane][4], wb[kRowsPerLane][4];
        if (n > 0 && live(0))
            load_plain(a, (int64_t)tm0 * kTileM + row_off, k, wa);
        for (int g = 0; g < n; g += 2) {
            if (g + 1 < n && live(g + 1))
                load_plain(a, (int64_t)(tm0 + g + 1) * kTileM + row_off, k, wb);
            tile_step<ROW, COL, DBIAS>(a, wa, srow, st, tm0 + g, tk, g, dsum);
            if (g + 1 < n) {
                if (g + 2 < n && live(g + 2))
                    load_plain(a, (int64_t)(tm0 + g + 2) * kTileM + row_off, k, wa);
                tile_step<ROW, COL, DBIAS>(a, wb, srow, st, tm0 + g + 1, tk, g + 1, dsum);
            }
        }
    } else {
        uint32_t w[kRowsPerLane][4];
        for (int g = 0; g < n; g++) {
            if (live(g)) {
                const int64_t m0 = (int64_t)(tm0 + g) * kTileM + row_off;
                const uint16_t *px = a.x + m0 * a.ldx + k;
                load_rows<OP>(a, px, OP == OP_DGELU ? a.aux + m0 * a.ldx + k : px, w);
            }
            tile_step<ROW, COL, DBIAS>(a, w, srow, st, tm0 + g, tk, g, dsum);
        }
    }
    if constexpr (COL)
        col_flush_s(a, *st, rg, tk, n);

    if constexpr (DBIAS) {
        // per-lane sums (rows in order, sub-tiles in order), then the 8
        // lane-halves of the workgroup in order: one fp32 partial per
        // (strip segment, column)
        __shared__ float4 red[2 * kWaves][kTileK / 4];
        const int slot = 2 * wave + half;
        red[slot][cl * 2] = make_float4(dsum[0], dsum[1], dsum[2], dsum[3]);
        red[slot][cl * 2 + 1] = make_float4(dsum[4], dsum[5], dsum[6], dsum[7]);
        __syncthreads();
        const int t = (int)threadIdx.x;   // one column of the strip per thread
        const int64_t kc = (int64_t)tk * kTileK + t;
        if (kc < a.K) {
            const float *flat = reinterpret_cast<const float *>(red);
            float acc = flat[t];
#pragma unroll
            for (int v = 1; v < 2 * kWaves; v++)
                acc += flat[v * kTileK + t];
            a.partials[(int64_t)rg * a.K + kc] = acc;
        }
    }
}

// dbias[k] = sum over strip segments t (in order) of partials[t][k].
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float *partials, int segments,
                                                           int64_t K, float *dbias)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K)
        return;
    float acc = 0.0f;
    for (int t = 0; t < segments; t++)
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
    const int blocks = a.groups_m * a.tiles_k;
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

hipError_t launch_dbias_reduce(const float *partials, int segments, int64_t K, float *dbias,
                               hipStream_t s)
{
    const int64_t blocks = (K + 255) / 256;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials,
                       segments, K, dbias);
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
