// nvfp4.hip -- NVFP4 quantize-transpose for gfx950, plus the tensor absmax
// pass its global scale needs.  The pages time NVFP4 quantize-transpose
// kernels ("NVFP4 2D quantize-transpose kernel" table of TransformerEngine
// PR 3291, and its 1D bf16 kernel listed under "Patched but not
// measurable"); this is the 1D form: 16-element blocks along K for the
// row-wise output and along M for the transposed output.
//
// Same work layout as the MXFP8 cast: a lane owns 16 rows x 8 columns of a
// 128 x 256 sub-tile, which makes each lane's 16 rows exactly one column
// block of the transposed output (no cross-lane work for dim1); a row block
// of 16 spans two lanes, combined with one DPP permute.  A workgroup walks
// down a 256-column strip with the next sub-tile's loads in flight; the
// transposed nibbles of two sub-tiles are staged in LDS and leave as whole
// 128-byte lines, the column scales of the whole walk at its end, the row
// scales of each sub-tile as 16-byte pieces.  All global access goes through
// buffer resources (bufio.h).
//
// Per block the scale chain costs three IEEE fp32 divisions (b/6, /S_g and
// the reciprocal); each element then costs one multiply and half of a packed
// hardware E2M1 convert.

#include "bufio.h"
#include "device_math.h"
#include "launch.h"
#include "nv_block.h"
#include "rag_flush.h"
#include "stage_flush.h"

namespace mxk {

// Rows 8q..8q+7 of one column (half HI of word d) times inv -> eight nibbles,
// row 8q+i in bits 4i..4i+3 (NaN products cleared as above).
template <int HI>
__device__ __forceinline__ uint32_t encode8_fp4_col(const uint32_t (&w)[kRowsPerLane][4], int q,
                                                    int d, float inv)
{
    auto h = [&](int i) { return HI ? w[8 * q + i][d] >> 16 : w[8 * q + i][d]; };
    auto v = [&](int i) { return (HI ? bf16_hi(w[8 * q + i][d]) : bf16_lo(w[8 * q + i][d])) * inv; };
    uint32_t o = e2m1x2<0>(v(0), v(1), 0u);
    o = e2m1x2<1>(v(2), v(3), o);
    o = e2m1x2<2>(v(4), v(5), o);
    o = e2m1x2<3>(v(6), v(7), o);
    const bool inf = __builtin_isinf(inv);
    if (__builtin_amdgcn_ballot_w64(inf) != 0) {
        uint32_t clear = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            clear |= zero_or_nan_nibble(h(i)) << (4 * i);
        o &= inf ? ~clear : ~0u;
    }
    return o;
}

// Cache policy of each stream (as for the MXFP8 cast): non-temporal input;
// with both outputs, non-temporal transposed output.
template <bool ROW, bool COL>
struct NvPolicy {
    static constexpr int x = kNT;
    static constexpr int q_row = 0, s_row = 0;
    static constexpr int q_col = ROW && COL ? kNT : 0;
    static constexpr int s_col = ROW && COL ? kNT : 0;
};

// Lane coordinates: the lane's 16 rows start at `row` inside the sub-tile.
struct NvLane {
    int wave, half, cl, row;
};

__device__ __forceinline__ NvLane nv_lane()
{
    NvLane l;
    l.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    l.half = lane >> 5;
    l.cl = lane & 31;
    l.row = l.wave * (2 * kRowsPerLane) + l.half * kRowsPerLane;
    return l;
}

// M and K are multiples of 16: a lane's 16 rows, and the two lanes of a row
// block, exist or not together.
__device__ __forceinline__ bool nv_live(const Nv4Args &a, const NvLane &l, int tm, int tk)
{
    return (int64_t)tm * kTileM + l.row < a.M && (int64_t)tk * kTileK + l.cl * kColsPerLane < a.K;
}

// LDS staging.  q: the transposed E2M1 output of two consecutive sub-tiles
// (256 rows = 128 bytes per transposed row), as 8 chunks of 16 bytes per
// transposed row, chunk j at position j ^ ((kl >> 3) & 7) (the flush reads a
// row's 8 chunks with 8 threads without bank conflicts).  Sub-tile p of the
// pair fills chunks 4p..4p+3; the lane of rows 16h..16h+15 of the sub-tile
// writes bytes 8 nv_half(kl, h & 1) of chunk 4p + h / 2.  s: the 8 column-block scales
// per sub-tile of the whole walk, transposed (block-major, stage_flush.h).
// srow: the 16 row-block scales per row of the current sub-tile.
// RAG (transposed rows at any byte, rag_flush.h): two pair tiles, the
// current pair's and the previous one's; walks of at most kMaxNvRagGroup
// sub-tiles keep the stage within two workgroups per CU.
template <bool RAG>
struct NvStageT {
    uint8_t q[RAG ? 2 : 1][kTileK][128];                        // 32 KB each
    uint8_t s[8 * (RAG ? kMaxNvRagGroup : kMaxGroup)][kTileK];  // 32 KB, 8 KB
    uint8_t srow[kTileM][kTileK / 16];                          // 2 KB
    float inv[128];                                             // multiplier of each scale byte
};
using NvStage = NvStageT<false>;

__device__ __forceinline__ int nv_chunk(int kl, int j) { return j ^ ((kl >> 3) & 7); }

// The 8-byte half of a staged chunk that rows 16h .. 16h + 15 of the wave
// (h = half) go to: swapped for transposed rows with bit 6 set, so that lanes
// cl and cl + 8 -- whose rows share a chunk position -- write different halves
// and any 16 consecutive lanes write 16 different 8-byte slots of a 128-byte
// span (no LDS bank conflict); the flush swaps them back.
__device__ __forceinline__ int nv_half(int kl, int half) { return half ^ ((kl >> 6) & 1); }

// Chunk j (0-7) of staged transposed row kr, its 8-byte halves in logical
// order: where the halves are swapped, the chunk's first 8 bytes lie in its
// second half, so the two 8-byte reads take them in that order (no selects).
__device__ __forceinline__ uint4 nv_read_chunk(const uint8_t *row, int kr, int j)
{
    const uint8_t *p = row + 16 * nv_chunk(kr, j);
    const int h = nv_half(kr, 0) ? 8 : 0;
    const uint2 lo = *reinterpret_cast<const uint2 *>(p + h);
    const uint2 hi = *reinterpret_cast<const uint2 *>(p + (8 - h));
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The staged pair tiles of a ragged walk as rag_flush.h reads them, each
// chunk's 8-byte halves back in order.
struct NvRagView {
    const uint8_t (*prev)[128], (*cur)[128];
    __device__ __forceinline__ uint4 chunk(int kr, int c) const
    {
        return nv_read_chunk(c < 8 ? prev[kr] : cur[kr], kr, c & 7);
    }
};

template <int XA>
__device__ __forceinline__ void nv_load(const Nv4Args &a, const NvLane &l, int tm, int tk,
                                        uint32_t (&w)[kRowsPerLane][4])
{
    const int64_t tile = (int64_t)tm * kTileM * a.K + (int64_t)tk * kTileK;
    const rsrc_t rx = make_rsrc(a.x, 2 * tile, 2 * a.M * a.K);
    const uint32_t rs = (uint32_t)(2 * a.K);
    const uint32_t off = nv_live(a, l, tm, tk)
                             ? (uint32_t)l.row * rs + (uint32_t)(2 * kColsPerLane * l.cl)
                             : kDead;
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        const uint4 v = buf_load16<XA>(rx, off + r * rs);
        w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
    }
}

// Transposed output of the staged pair (chunks 0..4 * parts - 1 of each
// transposed row; parts = 1 when the walk ends on the first sub-tile of a
// pair).  tm: the pair's first sub-tile.  half: M is not a multiple of 32,
// so a 16-byte chunk may hold 16 rows inside M and 16 outside; then each
// chunk leaves as two 8-byte halves (a run-time choice, so that the groups of
// a grouped cast each take their own).
template <int AUX, bool TWO_D>
__device__ __forceinline__ void nv_flush_q(const Nv4Args &a, const NvStage &st, int tm, int tk,
                                           int parts, bool half)
{
    const int t = (int)threadIdx.x;
    const int jr = t & 7;
    const int64_t m0 = (int64_t)tm * kTileM;
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t ld = a.M >> 1;                               // bytes per transposed row
    const rsrc_t rc = make_rsrc(a.q_col, k0 * ld + (m0 >> 1), a.K * ld);
    const int64_t row0 = m0 + 32 * jr;                         // first row of chunk jr
    const bool in_pair = jr < 4 * parts;
#pragma unroll
    for (int i = 0; i < kTileK / 32; i++) {
        const int kr = (t >> 3) + 32 * i;
        const bool col_ok = in_pair && k0 + kr < a.K;
        // the 2D casts read the halves in order; the 1D casts, short of
        // registers, read the chunk whole and swap its halves with selects
        // (4 more spilled registers and 2 % slower the other way round)
        uint4 v;
        if constexpr (TWO_D) {
            v = nv_read_chunk(st.q[0][kr], kr, jr);
        } else {
            v = *reinterpret_cast<const uint4 *>(&st.q[0][kr][16 * nv_chunk(kr, jr)]);
            if (nv_half(kr, 0))
                v = make_uint4(v.z, v.w, v.x, v.y);
        }
        const uint32_t off = (uint32_t)(kr * ld) + 16 * jr;
        if (!half) {
            buf_store16<AUX>(rc, col_ok && row0 < a.M ? off : kDead, v);
        } else {
            // rows of M / 2 bytes (M not a multiple of 32) do not start on
            // 16-byte boundaries: 8-byte pieces, completed in L2 with the
            // neighbouring chunks, so with the default cache policy
            buf_store8<0>(rc, col_ok && row0 < a.M ? off : kDead, make_uint2(v.x, v.y));
            buf_store8<0>(rc, col_ok && row0 + 16 < a.M ? off + 8 : kDead, make_uint2(v.z, v.w));
        }
    }
}

// Transposed output of pair pp of a walk whose transposed rows start at any
// byte (the tensor's M, or the rows before its group, not a multiple of 16):
// pairs are the steps of rag_flush_lines, rows of ceil(M/2) bytes.  tm: the
// pair's first sub-tile; parts 1: the pair holds that sub-tile only.
template <int AUX>
__device__ __forceinline__ void nv_flush_q_rag(const Nv4Args &a, const NvStageT<true> &st, int tm,
                                               int tk, int pp, int parts, bool first, bool last)
{
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t ld = (a.M + 1) >> 1;                        // bytes per transposed row
    const int64_t b0 = (int64_t)tm * (kTileM / 2);             // the pair's first byte of a row
    const int64_t cap = 64 * parts;
    const int rem = (int)(ld - b0 < cap ? ld - b0 : cap);
    // descriptor from the line boundary at or below the pair's first byte of
    // row k0; a row's offset d0 + kr ld is below 255 * 2^22 + 128
    const uint8_t *row0 = a.q_col + k0 * ld;
    const uint32_t d0 = (uint32_t)(reinterpret_cast<uintptr_t>(row0) & 127u);
    const rsrc_t rc = make_rsrc(row0 - d0, b0, (a.K - k0) * ld + d0);
    const NvRagView v{st.q[(pp & 1) ^ 1], st.q[pp & 1]};
    rag_flush_lines<AUX>(v, rc, d0, (uint32_t)ld, a.K - k0, rem, first, last);
}

// Column-block scales of the walk: 8 n bytes per column for n sub-tiles,
// 16-byte chunks from neighbouring threads when s_col's rows allow it.
template <int AUX, class Stage>
__device__ __forceinline__ void nv_flush_s(const Nv4Args &a, const Stage &st, int tm0, int tk,
                                           int n)
{
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t nblk = (a.M + 15) >> 4;                      // scales per column
    const int64_t first = (int64_t)tm0 * (kTileM / 16);
    const int64_t left = nblk - first;
    const int count = (int)(left < 8 * n ? left : 8 * n);
    const rsrc_t rs = make_rsrc(a.s_col, k0 * nblk + first, a.K * nblk);
    flush_scale_rows<AUX>(rs, st.s, k0, a.K, nblk, first, count, a.s_col);
}

// Row-block scales of sub-tile tm: thread t < 128 writes row t's 16 bytes.
template <int AUX, class Stage>
__device__ __forceinline__ void nv_flush_srow(const Nv4Args &a, const Stage &st, int tm, int tk)
{
    const int t = (int)threadIdx.x;
    const int64_t row = (int64_t)tm * kTileM + t;
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t nb = a.K >> 4;
    const rsrc_t rs = make_rsrc(a.s_row, (int64_t)tm * kTileM * nb + (k0 >> 4), a.M * nb);
    const uint32_t off = t < kTileM && row < a.M ? (uint32_t)(t * nb) : kDead;
    const uint8_t *src = st.srow[t & (kTileM - 1)];
    if ((a.K & 255) == 0) {
        buf_store16<AUX>(rs, off, *reinterpret_cast<const uint4 *>(src));
    } else {
        const int64_t blocks = nb - (k0 >> 4);
#pragma unroll
        for (int b = 0; b < kTileK / 16; b++)
            buf_store1<AUX>(rs, b < blocks ? off + b : kDead, src[b]);
    }
}

// One sub-tile (g-th of the walk): row blocks (direct stores, scales to
// LDS), column blocks into the staging pair; FLUSH 0: keep staging, 1: the
// walk ends on the first sub-tile of a pair, 2: the pair is complete.
// 2D scaling: the lane's 16 rows x 8 columns and its pair lane's form one
// 16 x 16 block; one scale and multiplier serve all its elements, in both
// outputs.
template <bool ROW, bool COL, bool RAG>
__device__ __forceinline__ void nv_step_2d(const Nv4Args &a, const NvLane &l,
                                           const uint32_t (&w)[kRowsPerLane][4], NvStageT<RAG> &st,
                                           const DivBy &sg, rsrc_t rq, uint32_t qoff, int g)
{
    using P = NvPolicy<ROW, COL>;
    uint32_t t = 0;
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++)
#pragma unroll
        for (int d = 0; d < 4; d++)
            t = pk_max_u16(t, w[r][d] & 0x7FFF7FFFu);
    const uint32_t lo = t & 0xFFFFu, hi = t >> 16;
    const uint32_t sb = nv_scale(max_xor1(lo > hi ? lo : hi), sg);
    const float inv = st.inv[sb];
    if constexpr (ROW) {
#pragma unroll
        for (int r = 0; r < kRowsPerLane; r++) {
            buf_store4<P::q_row>(rq, qoff + (uint32_t)(r * (a.K >> 1)), encode8_fp4(w[r], inv));
            if ((l.cl & 1) == 0)
                st.srow[l.row + r][l.cl >> 1] = (uint8_t)sb;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (COL) {
        // re-derive the fp32 values from the packed words (see nv_step)
        uint32_t wc[kRowsPerLane][4];
#pragma unroll
        for (int r = 0; r < kRowsPerLane; r++)
#pragma unroll
            for (int d = 0; d < 4; d++) {
                wc[r][d] = w[r][d];
                if constexpr (ROW)
                    asm volatile("" : "+v"(wc[r][d]));
            }
        const int jr = 4 * (g & 1) + l.wave;
#pragma unroll
        for (int c = 0; c < kColsPerLane; c++) {
            const int d = c >> 1;
            uint32_t o[2];
#pragma unroll
            for (int q = 0; q < 2; q++)
                o[q] = (c & 1) ? encode8_fp4_col<1>(wc, q, d, inv) : encode8_fp4_col<0>(wc, q, d, inv);
            const int kl = l.cl * kColsPerLane + c;
            *reinterpret_cast<uint2 *>(
                &st.q[RAG ? (g >> 1) & 1 : 0][kl][16 * nv_chunk(kl, jr) + 8 * nv_half(kl, l.half)]) =
                make_uint2(o[0], o[1]);
        }
        // the 16 x 16 block's scale, for each of the lane's 8 columns
        const uint32_t rep = sb * 0x01010101u;
        stage_scales8(st.s, 8 * g + 2 * l.wave + l.half, l.cl, make_uint2(rep, rep));
    }
}

template <bool ROW, bool COL, bool TWO_D, int FLUSH, bool RAG>
__device__ __forceinline__ void nv_step(const Nv4Args &a, const NvLane &l,
                                        const uint32_t (&w)[kRowsPerLane][4], NvStageT<RAG> &st,
                                        const DivBy &sg, int tm, int tk, int g, int n)
{
    using P = NvPolicy<ROW, COL>;
    const bool live = nv_live(a, l, tm, tk);
    uint32_t cmax[4] = {0u, 0u, 0u, 0u};
    rsrc_t rq;
    uint32_t qoff = kDead;
    if constexpr (ROW) {
        const int64_t ld = a.K >> 1;
        rq = make_rsrc(a.q_row, (int64_t)tm * kTileM * ld + (int64_t)tk * (kTileK / 2), a.M * ld);
        if (live)
            qoff = (uint32_t)(l.row * ld) + 4 * l.cl;
    }
    if constexpr (TWO_D) {
        nv_step_2d<ROW, COL, RAG>(a, l, w, st, sg, rq, qoff, g);
    } else {
    // Rows go in pairs: both lanes of a row block know the block maxima of
    // rows r and r + 1; the even lane derives the scale of row r, the odd
    // lane that of row r + 1, and they swap results.  The pairs go in two
    // batches of four: the four codes first (one division each, one pair at
    // a time: left alone, the scheduler interleaves the divisions of all rows
    // and runs out of registers), then their eight multipliers read from LDS
    // together -- one wait for LDS per batch rather than one per lookup.
    const bool odd = l.cl & 1;
#pragma unroll
    for (int r0 = 0; r0 < kRowsPerLane; r0 += kRowsPerLane / 2) {
        uint32_t mine[kRowsPerLane / 4];
#pragma unroll
        for (int r = r0; r < r0 + kRowsPerLane / 2; r += 2) {
            uint32_t mag2[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                uint32_t m[4];
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    m[d] = w[r + h][d] & 0x7FFF7FFFu;
                    if constexpr (COL)
                        cmax[d] = pk_max_u16(cmax[d], m[d]);
                }
                const uint32_t t = pk_max_u16(pk_max_u16(m[0], m[1]), pk_max_u16(m[2], m[3]));
                const uint32_t lo = t & 0xFFFFu, hi = t >> 16;
                mag2[h] = max_xor1(lo > hi ? lo : hi);
            }
            if constexpr (ROW)
                mine[(r - r0) >> 1] = nv_scale(odd ? mag2[1] : mag2[0], sg);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ROW) {
            float inv0[kRowsPerLane / 4], inv1[kRowsPerLane / 4];
#pragma unroll
            for (int p = 0; p < kRowsPerLane / 4; p++) {
                const uint32_t other =
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)mine[p], 0xB1, 0xF, 0xF, false);
                const uint32_t sb0 = odd ? other : mine[p], sb1 = odd ? mine[p] : other;
                inv0[p] = st.inv[sb0];
                inv1[p] = st.inv[sb1];
                if (!odd) {
                    st.srow[l.row + r0 + 2 * p][l.cl >> 1] = (uint8_t)sb0;
                    st.srow[l.row + r0 + 2 * p + 1][l.cl >> 1] = (uint8_t)sb1;
                }
            }
#pragma unroll
            for (int p = 0; p < kRowsPerLane / 4; p++) {
                const int r = r0 + 2 * p;
                buf_store4<P::q_row>(rq, qoff + (uint32_t)(r * (a.K >> 1)),
                                     encode8_fp4(w[r], inv0[p]));
                buf_store4<P::q_row>(rq, qoff + (uint32_t)((r + 1) * (a.K >> 1)),
                                     encode8_fp4(w[r + 1], inv1[p]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if constexpr (COL) {
        // The row pass expanded every element to fp32; without this empty,
        // register-only barrier the compiler keeps those 128 values alive for
        // reuse here instead of re-deriving them from the 64 packed words.
        uint32_t wc[kRowsPerLane][4];
#pragma unroll
        for (int r = 0; r < kRowsPerLane; r++)
#pragma unroll
            for (int d = 0; d < 4; d++) {
                wc[r][d] = w[r][d];
                if constexpr (ROW)
                    asm volatile("" : "+v"(wc[r][d]));
            }
        const int p = g & 1;
        const int jr = 4 * p + l.wave;                       // logical 16-byte chunk
        // the column codes in two batches of four, each batch's multipliers
        // read from LDS together
        uint32_t sbs[kColsPerLane];
#pragma unroll
        for (int c0 = 0; c0 < kColsPerLane; c0 += kColsPerLane / 2) {
            float inv[kColsPerLane / 2];
#pragma unroll
            for (int c = c0; c < c0 + kColsPerLane / 2; c++) {
                const int d = c >> 1, hi = c & 1;
                sbs[c] = nv_scale(hi ? (cmax[d] >> 16) : (cmax[d] & 0xFFFFu), sg);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int c = c0; c < c0 + kColsPerLane / 2; c++)
                inv[c - c0] = st.inv[sbs[c]];
#pragma unroll
            for (int c = c0; c < c0 + kColsPerLane / 2; c++) {
                const int d = c >> 1, hi = c & 1;
                const float v = inv[c - c0];
                uint32_t o[2];
#pragma unroll
                for (int q = 0; q < 2; q++)
                    o[q] = hi ? encode8_fp4_col<1>(wc, q, d, v) : encode8_fp4_col<0>(wc, q, d, v);
                const int kl = l.cl * kColsPerLane + c;
                *reinterpret_cast<uint2 *>(&st.q[RAG ? (g >> 1) & 1 : 0][kl][16 * nv_chunk(kl, jr) +
                                                                  8 * nv_half(kl, l.half)]) =
                    make_uint2(o[0], o[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        stage_scales8(st.s, 8 * g + 2 * l.wave + l.half, l.cl, pack8(sbs));
    }
    }
    __syncthreads();
    if constexpr (ROW)
        nv_flush_srow<P::s_row>(a, st, tm, tk);
    if constexpr (COL && FLUSH != 0 && RAG)
        nv_flush_q_rag<P::q_col>(a, st, FLUSH == 2 ? tm - 1 : tm, tk, g >> 1, FLUSH, g < 2,
                                 FLUSH == 1 || g + 1 == n);
    else if constexpr (COL && FLUSH != 0)
        nv_flush_q<P::q_col, TWO_D>(a, st, FLUSH == 2 ? tm - 1 : tm, tk, FLUSH, (a.M & 31) != 0);
    __syncthreads();
}

// A workgroup walks a 256-column strip down `group` sub-tiles of 128 rows,
// with the next sub-tile's loads in flight while one is converted (as in the
// MXFP8 cast); the transposed output leaves every second sub-tile as whole
// 128-byte lines.

// A tensor whose amax is not finite (it holds an Inf or a NaN) has no usable
// global scale: the walk's sub-tiles get scale bytes 0x7F (the E4M3 NaN) and
// element codes 0, in 8-byte pieces of element rows and single scale bytes,
// every piece outside the tensor dropped by its descriptor.
template <bool ROW, bool COL, bool RAG>
__device__ void nv_fill_nonfinite(const Nv4Args &a, int tm0, int n, int tk)
{
    const int t = (int)threadIdx.x;
    const int64_t k0 = (int64_t)tk * kTileK;
    const uint2 zero = make_uint2(0u, 0u);
    for (int g = 0; g < n; g++) {
        const int64_t m0 = (int64_t)(tm0 + g) * kTileM;
        if constexpr (ROW) {
            // 128 rows x (128 element bytes, 16 scale bytes)
            const int64_t lq = a.K >> 1, ls = a.K >> 4;
            const rsrc_t rq = make_rsrc(a.q_row, m0 * lq + (k0 >> 1), a.M * lq);
            const rsrc_t rs = make_rsrc(a.s_row, m0 * ls + (k0 >> 4), a.M * ls);
            for (int i = t; i < kTileM * 16; i += kThreads) {
                const int r = i >> 4, p = i & 15;
                const bool row_ok = m0 + r < a.M;
                buf_store8<0>(rq, row_ok && (k0 >> 1) + 8 * p < lq ? (uint32_t)(r * lq + 8 * p) : kDead,
                              zero);
                buf_store1<0>(rs, row_ok && (k0 >> 4) + p < ls ? (uint32_t)(r * ls + p) : kDead,
                              (uint8_t)0x7F);
            }
        }
        if constexpr (COL) {
            // 256 transposed rows x (64 element bytes, 8 scale bytes); rows
            // that start at any byte (RAG) take the element bytes one by one
            const int64_t lq = (a.M + 1) >> 1, ls = (a.M + 15) >> 4;
            const rsrc_t rq = make_rsrc(a.q_col, k0 * lq + (m0 >> 1), a.K * lq);
            const rsrc_t rs = make_rsrc(a.s_col, k0 * ls + (m0 >> 4), a.K * ls);
            for (int i = t; i < kTileK * 8; i += kThreads) {
                const int kr = i >> 3, p = i & 7;
                const bool row_ok = k0 + kr < a.K;
                if constexpr (RAG) {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        buf_store1<0>(rq, row_ok && (m0 >> 1) + 8 * p + e < lq
                                              ? (uint32_t)(kr * lq + 8 * p + e) : kDead,
                                      (uint8_t)0);
                } else {
                    buf_store8<0>(rq, row_ok && (m0 >> 1) + 8 * p < lq ? (uint32_t)(kr * lq + 8 * p)
                                                                     : kDead,
                                  zero);
                }
                buf_store1<0>(rs, row_ok && (m0 >> 4) + p < ls ? (uint32_t)(kr * ls + p) : kDead,
                              (uint8_t)0x7F);
            }
        }
    }
}

template <bool ROW, bool COL, bool TWO_D, bool RAG = false>
__device__ __forceinline__ void nv_walk(const Nv4Args &a, int rg, int tk)
{
    using P = NvPolicy<ROW, COL>;
    const int tm0 = rg * a.group;
    const int n = (a.tiles_m - tm0) < a.group ? (a.tiles_m - tm0) : a.group;
    const NvLane l = nv_lane();

    const float sgf = nv_global_scale(*a.amax);
    if (!__builtin_isfinite(sgf)) {   // uniform: every thread of the workgroup returns
        nv_fill_nonfinite<ROW, COL, RAG>(a, tm0, n, tk);
        return;
    }
    const DivBy sg = div_by_prepare(sgf);

    __shared__ NvStageT<RAG> st;
    if (threadIdx.x < 128)
        st.inv[threadIdx.x] = nv_inverse(threadIdx.x, sgf);
    __syncthreads();
    if constexpr (RAG) {
        // without the prefetch: its second register set would not fit
        // beside the two-pair flush at two workgroups per CU
        uint32_t w[kRowsPerLane][4];
        for (int g = 0; g < n; g++) {
            nv_load<P::x>(a, l, tm0 + g, tk, w);
            if (g & 1)
                nv_step<ROW, COL, TWO_D, 2, RAG>(a, l, w, st, sg, tm0 + g, tk, g, n);
            else if (g + 1 == n)
                nv_step<ROW, COL, TWO_D, 1, RAG>(a, l, w, st, sg, tm0 + g, tk, g, n);
            else
                nv_step<ROW, COL, TWO_D, 0, RAG>(a, l, w, st, sg, tm0 + g, tk, g, n);
        }
        if constexpr (COL)
            nv_flush_s<P::s_col>(a, st, tm0, tk, n);
        return;
    }
    uint32_t wa[kRowsPerLane][4], wb[kRowsPerLane][4];
    const int past = a.tiles_m;   // a sub-tile row outside the tensor: reads as zeros
    nv_load<P::x>(a, l, tm0, tk, wa);
    int g = 0;
    for (; g + 1 < n; g += 2) {
        nv_load<P::x>(a, l, tm0 + g + 1, tk, wb);
        __builtin_amdgcn_sched_barrier(0);
        nv_step<ROW, COL, TWO_D, 0, RAG>(a, l, wa, st, sg, tm0 + g, tk, g, n);
        nv_load<P::x>(a, l, g + 2 < n ? tm0 + g + 2 : past, tk, wa);
        __builtin_amdgcn_sched_barrier(0);
        nv_step<ROW, COL, TWO_D, 2, RAG>(a, l, wb, st, sg, tm0 + g + 1, tk, g + 1, n);
    }
    if (g < n)
        nv_step<ROW, COL, TWO_D, 1, RAG>(a, l, wa, st, sg, tm0 + g, tk, g, n);
    if constexpr (COL)
        nv_flush_s<P::s_col>(a, st, tm0, tk, n);
}

template <bool ROW, bool COL, bool TWO_D>
__global__ __launch_bounds__(kThreads, 2) void nvfp4_kernel(Nv4Args a)
{
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int rg = job / a.tiles_k;
    if (a.sg_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *a.sg_out = nv_global_scale(*a.amax);
    nv_walk<ROW, COL, TWO_D>(a, rg, job - rg * a.tiles_k);
}

// Grouped: walk rg (numbered across all groups) belongs to the group g with
// walk0[g] <= rg < walk0[g + 1], quantised as a tensor of its own with its
// own amax (amax[g]) and global scale.  Workgroup 0 writes every group's
// global scale (1 for an empty group).
template <bool ROW, bool COL, bool TWO_D, bool RAG>
__global__ __launch_bounds__(kThreads, 2) void nvfp4_grouped_kernel(Nv4Args a, GroupTable gt)
{
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int rg = job / a.tiles_k;
    const int tk = job - rg * a.tiles_k;
    if (a.sg_out != nullptr && blockIdx.x == 0 && (int)threadIdx.x < gt.count) {
        const int t = (int)threadIdx.x;
        a.sg_out[t] = gt.row0[t + 1] == gt.row0[t] ? 1.0f : nv_global_scale(a.amax[t]);
    }
    int g = 0;
    while (g + 1 < gt.count && gt.walk0[g + 1] <= rg)
        g++;
    const int64_t r0 = gt.row0[g];
    Nv4Args b = a;
    b.M = gt.row0[g + 1] - r0;
    b.x = a.x + r0 * a.K;
    b.amax = a.amax + g;
    b.q_row = a.q_row ? a.q_row + r0 * (a.K >> 1) : nullptr;
    b.s_row = a.s_row ? a.s_row + r0 * (a.K >> 4) : nullptr;
    // a group's transpose after the previous groups' [K][ceil(rows/2)] and
    // [K][ceil(rows/16)] bytes (the same as K r0 / 2 and K r0 / 16 when every
    // group's rows are a multiple of 16)
    b.q_col = a.q_col ? a.q_col + (RAG ? gt.qcol_off[g] : a.K * (r0 >> 1)) : nullptr;
    b.s_col = a.s_col ? a.s_col + (RAG ? gt.scol_off[g] : a.K * (r0 >> 4)) : nullptr;
    b.tiles_m = (int)((b.M + kTileM - 1) / kTileM);
    b.group = gt.len[g];
    b.groups_m = gt.walk0[g + 1] - gt.walk0[g];
    nv_walk<ROW, COL, TWO_D, RAG>(b, rg - gt.walk0[g], tk);
}

// ---------------------------------------------------------------------------
// Tensor absmax: largest |bf16| as the fp32 bit pattern (ordered like an
// unsigned integer for non-negative values), combined with atomic max.
// ---------------------------------------------------------------------------
__global__ void absmax_clear_kernel(uint32_t *amax_bits) { *amax_bits = 0u; }

// 16-byte vectors of the input through a global-address-space pointer, so the
// loads are global (not flat) loads; the input is read once, so they are
// non-temporal.
typedef const __attribute__((address_space(1))) u32x4_t gvec_t;

__device__ __forceinline__ uint32_t fold_vec(uint32_t m, u32x4_t v)
{
    return pk_max_u16(m, pk_max_u16(pk_max_u16(v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu),
                                    pk_max_u16(v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu)));
}

// Largest 15-bit magnitudes (two packed halves) of this workgroup's chunk of
// vectors, [b0, b1): each pass reads eight runs of 256 consecutive vectors
// (4 KiB each, one per wave instruction), eight independent loads in flight
// per thread.  A workgroup reading a contiguous chunk keeps its accesses in
// few DRAM pages; measured on the 16384^2 tensor, 512 chunked workgroups read
// at 6.1 TB/s against 5.1 TB/s for a grid-strided loop.
__device__ __forceinline__ uint32_t absmax_chunk(const uint16_t *x, int64_t b0, int64_t b1)
{
    gvec_t *xv = (gvec_t *)x;
    uint32_t m = 0;
    int64_t i = b0 + threadIdx.x;
    for (; i + 7 * 256 < b1; i += 8 * 256) {
        u32x4_t v[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = __builtin_nontemporal_load(xv + i + j * 256);
#pragma unroll
        for (int j = 0; j < 8; j++)
            m = fold_vec(m, v[j]);
    }
    for (; i < b1; i += 256)
        m = fold_vec(m, __builtin_nontemporal_load(xv + i));
    return m;
}

// Chunk of workgroup b of nb over nvec vectors.
__device__ __forceinline__ void chunk_of(int64_t nvec, int b, int nb, int64_t &b0, int64_t &b1)
{
    const int64_t per = (nvec + nb - 1) / nb;
    b0 = (int64_t)b * per;
    b1 = b0 + per < nvec ? b0 + per : nvec;
}

// The workgroup's largest magnitude, combined into *dst by one atomic max
// (of its fp32 bit pattern) from thread 0.
__device__ __forceinline__ void absmax_commit(uint32_t m, uint32_t *dst)
{
    uint32_t mag = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mag, off, 64);
        mag = mag > o ? mag : o;
    }
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = mag;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t w = red[0];
#pragma unroll
        for (int i = 1; i < 4; i++)
            w = w > red[i] ? w : red[i];
        atomicMax(dst, w << 16);
    }
}

constexpr int kAbsmaxBlocks = 512;   // two 256-thread workgroups per CU

__global__ __launch_bounds__(256) void absmax_kernel(const uint16_t *x, int64_t n,
                                                     uint32_t *amax_bits)
{
    const int64_t nvec = n >> 3;
    int64_t b0, b1;
    chunk_of(nvec, (int)blockIdx.x, (int)gridDim.x, b0, b1);
    uint32_t m = absmax_chunk(x, b0, b1);
    if (blockIdx.x == 0 && threadIdx.x < (n & 7))   // the last n % 8 elements
        m = pk_max_u16(m, x[(nvec << 3) + threadIdx.x] & 0x7FFFu);
    absmax_commit(m, amax_bits);
}

// Per-group absmax: group g's elements are x[row0[g] K .. row0[g + 1] K).
__global__ void absmax_clear_grouped_kernel(uint32_t *amax_bits, int G)
{
    if ((int)threadIdx.x < G)
        amax_bits[threadIdx.x] = 0u;
}

// Workgroups of the grouped absmax: group g gets blk0[g + 1] - blk0[g] of
// them, in proportion to its size, so that every workgroup reads a chunk of
// about the same length.
struct AbsmaxPlan {
    int blk0[kMaxGroups + 1];
};

// The group's workgroups split the whole 16-byte vectors inside its element
// range; its first workgroup also takes the elements before the first and
// after the last of them (fewer than 8 each; all of them when the range
// holds no whole vector).
__global__ __launch_bounds__(256) void absmax_grouped_kernel(const uint16_t *x, int64_t K,
                                                             GroupTable gt, AbsmaxPlan plan,
                                                             uint32_t *amax_bits)
{
    const int b = (int)blockIdx.x;
    int g = 0;
    while (g + 1 < gt.count && plan.blk0[g + 1] <= b)
        g++;
    const int64_t e0 = gt.row0[g] * K, e1 = gt.row0[g + 1] * K;
    const int64_t v0 = (e0 + 7) >> 3, v1 = e1 >> 3;         // whole vectors [v0, v1)
    int64_t b0, b1;
    chunk_of(v1 > v0 ? v1 - v0 : 0, b - plan.blk0[g], plan.blk0[g + 1] - plan.blk0[g], b0, b1);
    uint32_t m = absmax_chunk(x + 8 * v0, b0, b1);
    if (b == plan.blk0[g] && threadIdx.x < 14) {
        const int64_t head_end = 8 * v0 < e1 ? 8 * v0 : e1;
        const int64_t tail0 = 8 * v1 > head_end ? 8 * v1 : head_end;
        const int i = (int)threadIdx.x;
        const int64_t e = i < 7 ? e0 + i : tail0 + (i - 7);
        if (i < 7 ? e < head_end : e < e1)
            m = pk_max_u16(m, x[e] & 0x7FFFu);
    }
    absmax_commit(m, amax_bits + g);
}

hipError_t launch_absmax(const uint16_t *x, int64_t n, float *amax, hipStream_t s)
{
    uint32_t *bits = reinterpret_cast<uint32_t *>(amax);
    hipLaunchKernelGGL(absmax_clear_kernel, dim3(1), dim3(1), 0, s, bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    int64_t blocks = ((n >> 3) + 2047) / 2048;   // at least 2048 vectors per workgroup
    blocks = blocks > kAbsmaxBlocks ? kAbsmaxBlocks : (blocks < 1 ? 1 : blocks);
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n, bits);
    return hipGetLastError();
}

hipError_t launch_absmax_grouped(const uint16_t *x, int64_t K, const GroupTable &gt, float *amax,
                                 hipStream_t s)
{
    uint32_t *bits = reinterpret_cast<uint32_t *>(amax);
    hipLaunchKernelGGL(absmax_clear_grouped_kernel, dim3(1), dim3(kMaxGroups), 0, s, bits,
                       gt.count);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // about kAbsmaxBlocks workgroups in all, each group's share in
    // proportion to its rows (at least one for a group with rows)
    AbsmaxPlan plan;
    const int64_t M = gt.row0[gt.count];
    int total = 0;
    for (int g = 0; g < gt.count; g++) {
        plan.blk0[g] = total;
        const int64_t rows = gt.row0[g + 1] - gt.row0[g];
        const int64_t want = (rows * kAbsmaxBlocks + M - 1) / M;
        const int64_t cap = ((rows * K >> 3) + 2047) / 2048;   // >= 2048 vectors each
        total += rows == 0 ? 0 : (int)(want < 1 ? 1 : (want > cap ? (cap < 1 ? 1 : cap) : want));
    }
    plan.blk0[gt.count] = total;
    hipLaunchKernelGGL(absmax_grouped_kernel, dim3((unsigned)total), dim3(256), 0, s, x, K, gt,
                       plan, bits);
    return hipGetLastError();
}

template <bool ROW, bool COL, bool TWO_D, bool RAG>
static hipError_t launch_nv(const Nv4Args &a, const GroupTable *gt, hipStream_t s)
{
    const dim3 grid((unsigned)(a.groups_m * a.tiles_k));
    if (RAG || gt)
        hipLaunchKernelGGL((nvfp4_grouped_kernel<ROW, COL, TWO_D, RAG>), grid, dim3(kThreads), 0, s,
                           a, *gt);
    else
        hipLaunchKernelGGL((nvfp4_kernel<ROW, COL, TWO_D>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <bool TWO_D, bool RAG = false>
static hipError_t launch_nv_axis(unsigned axis, const Nv4Args &a, const GroupTable *gt,
                                 hipStream_t s)
{
    switch (axis) {
    case 1u:
        // row-wise alone has no transposed rows to align: never the RAG variant
        if constexpr (RAG)
            return hipErrorInvalidValue;
        else
            return launch_nv<true, false, TWO_D, false>(a, gt, s);
    case 2u: return launch_nv<false, true, TWO_D, RAG>(a, gt, s);
    case 3u: return launch_nv<true, true, TWO_D, RAG>(a, gt, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_nvfp4(unsigned axis, bool two_d, const Nv4Args &a, hipStream_t s)
{
    return two_d ? launch_nv_axis<true>(axis, a, nullptr, s)
                 : launch_nv_axis<false>(axis, a, nullptr, s);
}

hipError_t launch_nvfp4_grouped(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                                hipStream_t s)
{
    return two_d ? launch_nv_axis<true>(axis, a, &gt, s) : launch_nv_axis<false>(axis, a, &gt, s);
}

hipError_t launch_nvfp4_ragged(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                               hipStream_t s)
{
    return two_d ? launch_nv_axis<true, true>(axis, a, &gt, s)
                 : launch_nv_axis<false, true>(axis, a, &gt, s);
}

}  // namespace mxk
