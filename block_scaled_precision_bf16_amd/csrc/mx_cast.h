// mx_cast.h -- the MXFP8 cast kernel for gfx950: row-wise (dim0), column-wise
// (dim1, transposed output) or both in one pass over the bf16 input,
// optionally with a fused GELU / dGELU / dSiLU / SwiGLU / GeGLU / dSwiGLU /
// dGeGLU pre-op and a dbias column sum, for one tensor or for a group of
// tensors stacked along M.  These are the kernels the TransformerEngine PR 3291 page
// times ("MXFP8 generic quantize kernel", "MXFP8 specialized cast-only kernel
// (bidimensional)", "MXFP8 gated (swiglu / geglu) kernel") and the torchao
// dim1 cast of PR 12, designed here for CDNA4.
//
// Layout of the work: a workgroup (4 waves) converts a 128-row x 256-column
// sub-tile at a time and walks down a 256-column strip.  A lane owns 16
// consecutive rows x 8 consecutive columns, loaded as 16 128-bit loads;
// lanes 0-31 of a wave hold rows 0-15 and lanes 32-63 rows 16-31 of the same
// 256 columns, so each wave load instruction reads two 512-byte row segments
// and a wave covers exactly one 32-row column block.  The row-wise amax spans
// 4 lanes (4 x 8 = 32 columns), reduced with two DPP quad permutes; row
// outputs leave as 8-byte stores (256 contiguous bytes per half-wave).  The
// column-wise amax of a column is the max of two lanes' in-register maxima
// (one exchange between lane l and l^32); each lane converts its own 16
// bytes of each transposed row into an LDS staging tile, from which the
// workgroup writes whole 128-byte lines of the transposed tensor.  Row and
// column scales are staged in LDS as well and leave as 8-byte and 16-byte
// pieces.  The LDS arrays are statically declared, so their addresses never
// pass through an integer (the fix the PR 3291 page is about).
//
// Every element costs a packed integer clamp and half of a packed scaled
// convert that applies the block's power-of-two scale exactly (the torchao
// PR 12 page: divisions per element made the dim1 cast compute bound; here
// there is not even a multiply per element).  All global memory access goes
// through buffer resources with out-of-range offsets for masked lanes (see
// bufio.h), so the load of the next sub-tile stays in flight while the
// current one is converted.
//
// The element format and the scale rule (E4M3 or E5M2; floor or round-up
// E8M0) are a template flag FMT; each of the four formats is instantiated
// in a translation unit of its own, plain (mx_cast_fmt_*.hip) and grouped
// (mx_cast_grp_*.hip), which keeps the build parallel.  The scale layout
// (compact or GEMM-ready tiles) is a run-time choice of the two flushes.
#pragma once

#include "bufio.h"
#include "device_math.h"
#include "launch.h"
#include "rag_flush.h"
#include "stage_flush.h"

namespace mxk {

__device__ __forceinline__ float half_value(uint32_t w, int hi)
{
    return hi ? bf16_hi(w) : bf16_lo(w);
}

// Cache policy of each stream, chosen by measurement (the 16384 x 16384 plain
// casts, the 8192 x 8192 fused ones).  The input is read once, so its loads
// are non-temporal, also for the dGELU, dSiLU and dSwiGLU casts, which read a
// grad stream beside it (3-5% faster there; 3-10% slower for GELU, dGeGLU and
// the forward gated casts).
// The row-wise elements of the plain casts are written with the SC1 bit.
// With both outputs the transposed tile (lines and scales) is written
// non-temporal as well; the row scales keep the default policy (non-temporal
// row scales, 8-byte pieces of lines that other workgroups complete, cost
// ~15%), and so does the transposed output alone (non-temporal: 26% slower).
// The policies change timing only, never results.
template <int OP, bool ROW, bool COL>
struct Policy {
    static constexpr bool plain = OP == OP_PLAIN, both = plain && ROW && COL;
    static constexpr int x =                              // input (and grad) loads
        plain || OP == OP_DGELU || OP == OP_DSILU || OP == OP_DSWIGLU ? kNT : 0;
    static constexpr int q_row = plain ? kSC1 : 0;       // row-wise stores
    static constexpr int s_row = 0;
    static constexpr int q_col = both ? kNT : 0;         // transposed stores
    static constexpr int s_col = both ? kNT : 0;
};

// Row r's 8 elements (4 words w, magnitudes mag) with scale byte b -> 8
// element bytes of format FMT.
template <int FMT>
__device__ __forceinline__ uint2 encode8_row(const uint32_t (&w)[4], const uint32_t (&mag)[4],
                                             uint32_t b)
{
    const uint32_t lim = sat_limit2<FMT>(b);
    const float sc = e8m0_operand(b);
    uint2 o;
    o.x = mx_pair<FMT, false>(w[0], mag[0], lim, sc, 0u);
    o.x = mx_pair<FMT, true>(w[1], mag[1], lim, sc, o.x);
    o.y = mx_pair<FMT, false>(w[2], mag[2], lim, sc, 0u);
    o.y = mx_pair<FMT, true>(w[3], mag[3], lim, sc, o.y);
    return o;
}

// Rows 2i and 2i+1 of one column (half HI of word d) as a packed bf16 pair.
template <int HI>
__device__ __forceinline__ uint32_t col_pair(const uint32_t (&w)[kRowsPerLane][4], int i, int d)
{
    return __builtin_amdgcn_perm(w[2 * i + 1][d], w[2 * i][d], HI ? 0x07060302u : 0x05040100u);
}

// One column's 16 rows (half HI of word d) with scale byte b -> 16 element
// bytes of format FMT, row 0 in the lowest byte.
template <int FMT, int HI>
__device__ __forceinline__ uint4 encode16_col(const uint32_t (&w)[kRowsPerLane][4], int d,
                                              uint32_t b)
{
    const uint32_t lim = sat_limit2<FMT>(b);
    const float sc = e8m0_operand(b);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t p0 = col_pair<HI>(w, 2 * j, d), p1 = col_pair<HI>(w, 2 * j + 1, d);
        const uint32_t t = mx_pair<FMT, false>(p0, p0 & 0x7FFF7FFFu, lim, sc, 0u);
        o[j] = mx_pair<FMT, true>(p1, p1 & 0x7FFF7FFFu, lim, sc, t);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Per-lane coordinates inside a sub-tile.
struct LaneAt {
    int wave, half, cl;
    int row;        // first of the lane's 16 rows inside the sub-tile
};

__device__ __forceinline__ LaneAt lane_at()
{
    LaneAt l;
    l.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = (int)threadIdx.x & 63;
    l.half = lane >> 5;
    l.cl = lane & 31;
    l.row = l.wave * (2 * kRowsPerLane) + l.half * kRowsPerLane;
    return l;
}

// The lane's wave has rows inside the tensor and its 8 columns exist (K is a
// multiple of 8, so a column group of 8 is wholly inside or outside).  Rows
// of a live wave past M (M is a multiple of 16) read as zeros and their
// stores fall outside the output's descriptor; a partial 32-column or 32-row
// block at the tensor's edge thus sees zeros for its missing elements, which
// change neither its amax nor any code.
__device__ __forceinline__ bool lane_live(const MxArgs &a, const LaneAt &l, int tm, int tk)
{
    return (int64_t)tm * kTileM + l.wave * 32 < a.M && (int64_t)tk * kTileK + l.cl * kColsPerLane < a.K;
}

// This lane's 16 rows x 8 columns of sub-tile (tm, tk), after the pre-op.  A
// sub-tile outside the tensor (tm >= tiles_m) reads as zeros without memory
// traffic, which the plain cast uses for the prefetch past a walk's end.
// HALF (gated backward): 1 when the whole sub-tile lies in the d_gate half,
// 0 when it lies in the d_linear half (the compiler then drops the other
// half's arithmetic), 2 when it straddles them.
template <int OP, int XA, int HALF = 2>
__device__ __forceinline__ void load_tile(const MxArgs &a, const LaneAt &l, int tm, int tk,
                                          uint32_t (&w)[kRowsPerLane][4])
{
    const bool live = lane_live(a, l, tm, tk);
    if constexpr (OP == OP_DSWIGLU || OP == OP_DGEGLU) {
        // output column k of [d_gate | d_linear] (each half N = lin_off wide)
        // reads gate and grad at column n = k mod N, and, in the gate half,
        // linear at N + n; a lane's 8 columns lie in one half (N % 8 == 0)
        const int64_t N = a.lin_off;
        const int64_t k = (int64_t)tk * kTileK + kColsPerLane * l.cl;
        const bool gate_half = HALF == 2 ? k < N : HALF == 1;
        const uint32_t n = (uint32_t)(gate_half ? k : k - N);
        const int64_t m0 = (int64_t)tm * kTileM;
        const rsrc_t rx = make_rsrc(a.x, 2 * m0 * a.ldx, 2 * a.M * a.ldx);
        const rsrc_t rg = make_rsrc(a.aux, 2 * m0 * a.ldg, 2 * a.M * a.ldg);
        // the linear half gets a descriptor of its own, based at column N of
        // the sub-tile's first row, and the gate's offsets: added to the
        // offset instead, the 2N bytes would take the last row's loads past
        // 2^31 - 1 (the largest descriptor) at 2N = 2^23
        const rsrc_t rl = make_rsrc(a.x, 2 * (m0 * a.ldx + N), 2 * a.M * a.ldx);
        const uint32_t sx = (uint32_t)(2 * a.ldx), sg = (uint32_t)(2 * a.ldg);
        const uint32_t ox = live ? (uint32_t)l.row * sx + 2 * n : kDead;
        const uint32_t og = live ? (uint32_t)l.row * sg + 2 * n : kDead;
        const uint32_t ol = live && gate_half ? ox : kDead;
#pragma unroll
        for (int r = 0; r < kRowsPerLane; r++) {
            const uint4 g = buf_load16<XA>(rx, ox + r * sx);
            const uint4 dy = buf_load16<XA>(rg, og + r * sg);
            const uint4 li = buf_load16<XA>(rl, ol + r * sx);
            w[r][0] = dgated_pair<OP>(g.x, dy.x, li.x, gate_half);
            w[r][1] = dgated_pair<OP>(g.y, dy.y, li.y, gate_half);
            w[r][2] = dgated_pair<OP>(g.z, dy.z, li.z, gate_half);
            w[r][3] = dgated_pair<OP>(g.w, dy.w, li.w, gate_half);
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    const int64_t tile = (int64_t)tm * kTileM * a.ldx + (int64_t)tk * kTileK;   // elements
    const int64_t total = a.M * a.ldx;
    const rsrc_t rx = make_rsrc(a.x, 2 * tile, 2 * total);
    const uint32_t rs = (uint32_t)(2 * a.ldx);
    const uint32_t off = live ? (uint32_t)l.row * rs + (uint32_t)(2 * kColsPerLane * l.cl) : kDead;
    rsrc_t rb = rx;
    uint32_t rbs = rs, boff = off;
    if constexpr (OP == OP_DGELU || OP == OP_DSILU) {
        const int64_t gtile = (int64_t)tm * kTileM * a.ldg + (int64_t)tk * kTileK;
        rb = make_rsrc(a.aux, 2 * gtile, 2 * a.M * a.ldg);
        rbs = (uint32_t)(2 * a.ldg);
        boff = live ? (uint32_t)l.row * rbs + (uint32_t)(2 * kColsPerLane * l.cl) : kDead;
    } else if constexpr (OP == OP_SWIGLU || OP == OP_GEGLU) {
        rb = make_rsrc(a.x, 2 * (tile + a.lin_off), 2 * total);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerLane; r++) {
        const uint4 v = buf_load16<XA>(rx, off + r * rs);
        if constexpr (OP == OP_PLAIN) {
            w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        } else {
            uint4 b = v;   // GELU has no second operand
            if constexpr (OP != OP_GELU)
                b = buf_load16<XA>(rb, boff + r * rbs);
            w[r][0] = fused_pair<OP>(v.x, b.x);
            w[r][1] = fused_pair<OP>(v.y, b.y);
            w[r][2] = fused_pair<OP>(v.z, b.z);
            w[r][3] = fused_pair<OP>(v.w, b.w);
            // one row's activation math at a time: interleaving rows only
            // multiplies the live temporaries
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Row-wise blocks of this lane's 16 rows: amax over 4 lanes x 8 columns,
// scale, convert, store.  Column maxima are accumulated on the way.
template <int OP, int FMT, bool ROW, bool COL>
__device__ __forceinline__ void row_pass(const MxArgs &a, const uint32_t (&w)[kRowsPerLane][4],
                                         const LaneAt &l, int tm, int tk, bool live, uint8_t *srow,
                                         uint32_t (&cmax)[4])
{
    rsrc_t rq;
    uint32_t off = kDead;
    if constexpr (ROW) {
        rq = make_rsrc(a.q_row, (int64_t)tm * kTileM * a.K + (int64_t)tk * kTileK, a.M * a.K);
        if (live)
            off = (uint32_t)(l.row * a.K) + (uint32_t)(kColsPerLane * l.cl);
    }
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
            const uint32_t sb = scale_byte<FMT>(mag);
            uint2 o = encode8_row<FMT>(w[r], m, sb);
            if (sb == 0xFFu)
                o.x = o.y = 0x7F7F7F7Fu;
            buf_store8<Policy<OP, ROW, COL>::q_row>(rq, off + (uint32_t)(r * a.K), o);
            if ((l.cl & 3) == 0)
                srow[r * (kTileK / 32)] = (uint8_t)sb;
        }
    }
}

// LDS staging of the column-wise output.  q: one sub-tile's transposed E4M3
// tile, q_col rows k0..k0+255, 128 bytes each (sub-tile rows m..m+127), as 8
// chunks of 16 bytes; chunk j of row kl is stored at chunk position
// j ^ ((kl >> 3) & 7): the 32 lanes of a half-wave write rows 8 apart (one
// per lane), the 8 threads that read a row back read its 8 chunks, and both
// patterns then cover all banks.  s: the column-block scales of the whole
// strip segment the workgroup walks (4 per sub-tile), transposed (block-major,
// stage_flush.h) and written out once.  RAG (transposed rows at any byte):
// two q tiles, the current sub-tile's and the previous one's, whose last
// bytes complete the first line the current one writes; walks of at most
// kMaxRagGroup sub-tiles keep the stage within two workgroups per CU.
template <bool RAG>
struct ColStageT {
    uint4 q[RAG ? 2 : 1][kTileK][kTileM / 16];                 // 32 KB each
    uint8_t s[4 * (RAG ? kMaxRagGroup : kMaxGroup)][kTileK];  // 16 KB, 14 KB
};
using ColStage = ColStageT<false>;
using StageTile = uint4[kTileK][kTileM / 16];

__device__ __forceinline__ int stage_chunk(int kl, int j) { return j ^ ((kl >> 3) & 7); }

// Column-wise blocks of sub-tile g: the 32 rows of a column block are this
// lane's 16 and those of lane l ^ 32; each lane converts its own 16 bytes of
// each column and puts them into the staging tile.
template <int FMT, bool RAG>
__device__ __forceinline__ void col_pass(ColStageT<RAG> &st, const uint32_t (&w)[kRowsPerLane][4],
                                         int wave, int half, int cl, int g, uint32_t (&cmax)[4])
{
#pragma unroll
    for (int d = 0; d < 4; d++)
        cmax[d] = pk_max_u16(cmax[d], (uint32_t)__shfl_xor((int)cmax[d], 32, 64));
    uint32_t sbs[kColsPerLane];
#pragma unroll
    for (int c = 0; c < kColsPerLane; c++) {
        const int d = c >> 1, hi = c & 1;
        const uint32_t mag = hi ? (cmax[d] >> 16) : (cmax[d] & 0xFFFFu);
        const uint32_t sb = scale_byte<FMT>(mag);
        uint4 o = hi ? encode16_col<FMT, 1>(w, d, sb) : encode16_col<FMT, 0>(w, d, sb);
        if (sb == 0xFFu)
            o = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
        const int kl = cl * kColsPerLane + c;
        st.q[RAG ? (g & 1) : 0][kl][stage_chunk(kl, 2 * wave + half)] = o;
        sbs[c] = sb;
    }
    // both halves hold the same column scales; one writes them
    if (half == 0)
        stage_scales8(st.s, 4 * g + wave, cl, pack8(sbs));
}

// Write the staged transposed tile of sub-tile tm: thread t writes 16-byte
// chunk t % 8 of q_col rows t / 8 + 32 i (i = 0..7), so each wave store
// instruction covers 8 whole 128-byte lines.
template <int AUX>
__device__ __forceinline__ void col_flush_q(const MxArgs &a, const ColStage &st, int tm, int tk)
{
    const int t = (int)threadIdx.x;
    const int jr = t & 7;
    const int64_t mt = (int64_t)tm * kTileM;
    const int64_t k0 = (int64_t)tk * kTileK;
    const rsrc_t rc = make_rsrc(a.q_col, k0 * a.M + mt, a.K * a.M);
    const bool chunk_live = mt + 16 * jr < a.M;   // M is a multiple of 16
#pragma unroll
    for (int i = 0; i < kTileK / 32; i++) {
        const int kr = (t >> 3) + 32 * i;
        const uint32_t off = chunk_live && k0 + kr < a.K ? (uint32_t)(kr * a.M) + 16 * jr : kDead;
        buf_store16<AUX>(rc, off, st.q[0][kr][stage_chunk(kr, jr)]);
    }
}

// The staged transposed tiles of a ragged MXFP8 walk, as rag_flush.h reads
// them: prev (the previous sub-tile's) and cur.
struct MxRagView {
    const StageTile &prev, &cur;
    __device__ __forceinline__ uint4 chunk(int kr, int c) const
    {
        // chunk c & 7 of the previous tile (c < 8) or of the current one
        const StageTile &tile = c < 8 ? prev : cur;
        return tile[kr][stage_chunk(kr, c & 7)];
    }
};

// The staged transposed tile of sub-tile g of a walk whose transposed rows
// start at any byte (the tensor's M, or the rows before its group, not a
// multiple of 16): sub-tiles are the steps of rag_flush_lines.
template <int AUX>
__device__ __forceinline__ void col_flush_q_rag(const MxArgs &a, const ColStageT<true> &st, int tm,
                                                int tk, int g, bool first, bool last)
{
    const int64_t mt = (int64_t)tm * kTileM;
    const int64_t k0 = (int64_t)tk * kTileK;
    const int rem = a.M - mt < kTileM ? (int)(a.M - mt) : kTileM;   // the sub-tile's bytes per row
    // descriptor from the line boundary at or below this sub-tile's first byte
    // of row k0; a row's offset d0 + kr M is below 255 * 2^23 + 128
    const uint8_t *row0 = a.q_col + k0 * a.M;
    const uint32_t d0 = (uint32_t)(reinterpret_cast<uintptr_t>(row0) & 127u);
    const rsrc_t rc = make_rsrc(row0 - d0, mt, (a.K - k0) * a.M + d0);
    const MxRagView v{st.q[(g & 1) ^ 1], st.q[g & 1]};
    rag_flush_lines<AUX>(v, rc, d0, (uint32_t)a.M, a.K - k0, rem, first, last);
}

// The 4-byte word lane L of a GEMM-ready scale tile holds: bytes j = 0..3 are
// blocks 2j + L / 32 of the tile's row L % 32, picked from that row's 8 staged
// block bytes (v.x = blocks 0-3, v.y = blocks 4-7).
__device__ __forceinline__ uint32_t tile_word(uint2 v, int lane)
{
    return __builtin_amdgcn_perm(v.y, v.x, (lane >> 5) ? 0x07050301u : 0x06040200u);
}

// Column scales of the strip segment in the GEMM-ready tile layout (tiles of
// 32 transposed rows x 8 blocks, 256 bytes, block-tile-major).  A walk starts
// on a tile boundary (its length is even), so its 4 n blocks per column fill
// whole tiles except, for odd n, the upper half of the last one, which holds
// no block of the tensor and is written as zeros.  The strip's 256
// transposed rows are 8 row tiles, contiguous for each block tile.
template <int AUX, class Stage>
__device__ __forceinline__ void col_flush_s_tiled(const MxArgs &a, const Stage &st, int rg,
                                                  int tk, int n)
{
    const int t = (int)threadIdx.x;
    const int64_t RT = (a.K + 31) >> 5;                   // row tiles of s_col
    const int64_t CT = (((a.M + 31) >> 5) + 7) >> 3;      // block tiles
    const int64_t bt0 = (int64_t)rg * (a.group >> 1);     // first block tile of the walk
    const int64_t rt0 = (int64_t)tk * (kTileK / 32);
    const int nbt = (4 * n + 7) >> 3;
    const rsrc_t rs = make_rsrc(a.s_col, (bt0 * RT + rt0) * 256, RT * CT * 256);
    for (int i = 0; i < 2 * nbt; i++) {
        const int idx = t + kThreads * i;                 // (block tile, row tile, lane)
        const int btl = idx >> 9, rtl = (idx >> 6) & 7, lane = idx & 63;
        uint32_t b8[2];
        staged_bytes<8>(st.s, 8 * btl, 32 * rtl + (lane & 31), b8);
        uint2 v = make_uint2(b8[0], b8[1]);
        if (4 * n - 8 * btl < 8)
            v.y = 0u;
        const uint32_t off = rt0 + rtl < RT ? (uint32_t)(((int64_t)btl * RT + rtl) * 256 + 4 * lane)
                                            : kDead;
        buf_store4<AUX>(rs, off, tile_word(v, lane));
    }
}

// Write the strip segment's column scales: 4 n bytes per column for a walk
// of n sub-tiles (the tile layout, or compact rows in the widest pieces the
// row length of s_col, the segment's start and its length allow).
template <int AUX, class Stage>
__device__ __forceinline__ void col_flush_s(const MxArgs &a, const Stage &st, int rg, int tk,
                                            int n)
{
    if (a.tiled) {
        col_flush_s_tiled<AUX>(a, st, rg, tk, n);
        return;
    }
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t nblk = (a.M + 31) >> 5;                 // scales per column
    const int64_t first = (int64_t)rg * a.group * 4;      // this segment's first block
    const int64_t left = nblk - first;
    const int count = (int)(left < 4 * n ? left : 4 * n);
    const rsrc_t rs = make_rsrc(a.s_col, k0 * nblk + first, a.K * nblk);
    flush_scale_rows<AUX>(rs, st.s, k0, a.K, nblk, first, count, a.s_col);
}

// Row scales of a sub-tile, staged as [128 rows][8 blocks] bytes: thread
// t < 128 writes row t's 8 scale bytes with one 8-byte store (instead of 8
// one-byte stores from 8 lanes).
template <int AUX>
__device__ __forceinline__ void srow_flush(const MxArgs &a, const uint8_t (&srow)[kTileM][kTileK / 32],
                                           int tm, int tk)
{
    const int t = (int)threadIdx.x;
    if (a.tiled) {
        // GEMM-ready layout: the sub-tile's 128 rows x 8 blocks are the four
        // 256-byte tiles (block tile tk, row tiles 4 tm .. 4 tm + 3), which
        // lie next to each other; thread t writes word t (tile t / 64, lane
        // t % 64).  Rows of a tile past M hold zero scales (padding).
        const int64_t RT = (a.M + 31) >> 5;
        const int64_t bytes = RT * ((((a.K + 31) >> 5) + 7) >> 3) * 256;
        const rsrc_t rs = make_rsrc(a.s_row, ((int64_t)tk * RT + 4 * (int64_t)tm) * 256, bytes);
        const int w = t >> 6, lane = t & 63;
        const uint2 v = *reinterpret_cast<const uint2 *>(srow[32 * w + (lane & 31)]);
        const bool live = (int64_t)tm * kTileM + 32 * w < a.M;
        buf_store4<AUX>(rs, live ? (uint32_t)(4 * t) : kDead, tile_word(v, lane));
        return;
    }
    const int64_t row = (int64_t)tm * kTileM + t;
    const int64_t k0 = (int64_t)tk * kTileK;
    const int64_t nb = (a.K + 31) >> 5;                   // scale bytes per row
    const rsrc_t rs = make_rsrc(a.s_row, (int64_t)tm * kTileM * nb + (k0 >> 5), a.M * nb);
    const uint32_t off = t < kTileM && row < a.M ? (uint32_t)(t * nb) : kDead;
    const uint8_t *src = srow[t & (kTileM - 1)];
    if ((a.K & 255) == 0) {
        buf_store8<AUX>(rs, off, *reinterpret_cast<const uint2 *>(src));
    } else {
        const int64_t blocks = nb - (k0 >> 5);            // scale bytes of this tile inside K
#pragma unroll
        for (int b = 0; b < kTileK / 32; b++)
            buf_store1<AUX>(rs, b < blocks ? off + b : kDead, src[b]);
    }
}

// One sub-tile of the walk: row pass (direct row stores, row scales to LDS),
// column pass into LDS, then the staged output leaves as whole lines.  Lanes
// outside the tensor hold zeros and their stores are out of range.
template <int OP, int FMT, bool ROW, bool COL, bool DBIAS, bool RAG>
__device__ __forceinline__ void tile_step(const MxArgs &a, const LaneAt &l,
                                          const uint32_t (&w)[kRowsPerLane][4],
                                          uint8_t (&srow)[kTileM][kTileK / 32],
                                          ColStageT<RAG> *st, int tm, int tk, int g, int n,
                                          float (&dsum)[kColsPerLane])
{
    const bool live = lane_live(a, l, tm, tk);
    uint32_t cmax[4] = {0u, 0u, 0u, 0u};
    row_pass<OP, FMT, ROW, COL>(a, w, l, tm, tk, live, &srow[l.row][l.cl >> 2], cmax);
    if constexpr (COL)
        col_pass<FMT, RAG>(*st, w, l.wave, l.half, l.cl, g, cmax);
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
    __syncthreads();
    if constexpr (COL && RAG) {
        col_flush_q_rag<Policy<OP, ROW, COL>::q_col>(a, *st, tm, tk, g, g == 0, g + 1 == n);
    } else if constexpr (COL) {
        // the non-temporal transposed stores pay off only for outputs too
        // large to be absorbed by the caches (the host decides: qcol_nt)
        if (Policy<OP, ROW, COL>::q_col == kNT && !a.qcol_nt)
            col_flush_q<0>(a, *st, tm, tk);
        else
            col_flush_q<Policy<OP, ROW, COL>::q_col>(a, *st, tm, tk);
    }
    if constexpr (ROW)
        srow_flush<Policy<OP, ROW, COL>::s_row>(a, srow, tm, tk);
    __syncthreads();   // the staging buffers are reused by the next sub-tile
}

// A workgroup walks a strip of 256 columns down `group` sub-tiles of 128 rows.
// Walking keeps the strip's column scales together (so they leave as whole
// 64-byte chunks rather than 4-byte pieces) and, for the plain cast, lets the
// next sub-tile's loads overlap the current sub-tile's conversion.
// Workgroups per CU the compiler budgets registers for: the fused casts
// without dbias are bound by their arithmetic and gain from a third
// workgroup (at most 168 VGPRs); the plain cast keeps its double register set
// for the prefetch, and the dbias sums and the gated backward need their
// registers (capping them spills and measured slower).
template <int OP, bool DBIAS, bool RAG = false>
constexpr int min_blocks()
{
    const int n = OP == OP_PLAIN || OP == OP_DSWIGLU || OP == OP_DGEGLU || DBIAS ? 1 : 3;
    // RAG: the double stage fits two workgroups per CU, and the plain cast
    // (without its prefetch there) takes two as well
    if (RAG)
        return n == 3 || (OP == OP_PLAIN && !DBIAS) ? 2 : n;
    return n;
}

// Walk rg of strip tk: the whole of a workgroup's work.
template <int OP, int FMT, bool ROW, bool COL, bool DBIAS, bool RAG = false>
__device__ __forceinline__ void mx_cast_walk(const MxArgs &a, int rg, int tk)
{
    const int tm0 = rg * a.group;
    const int n = (a.tiles_m - tm0) < a.group ? (a.tiles_m - tm0) : a.group;
    const LaneAt l = lane_at();

    __shared__ __align__(16) uint8_t srow[kTileM][kTileK / 32];
    ColStageT<RAG> *st = nullptr;
    if constexpr (COL) {
        __shared__ ColStageT<RAG> stage;
        st = &stage;
    }
    float dsum[kColsPerLane] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    if constexpr (OP == OP_PLAIN && !RAG) {
        // Software pipeline over two register sets (not with RAG: its second
        // register set beside the two-tile flush left one workgroup per CU,
        // slower than two without it).  Every pass through the
        // loop body issues the same memory instructions (the load past the
        // walk's end reads a sub-tile outside the tensor, which costs no
        // traffic), so the loads of the next sub-tile are never waited for
        // early; the scheduling barriers keep each prefetch where it is
        // issued instead of next to its first use.
        uint32_t wa[kRowsPerLane][4], wb[kRowsPerLane][4];
        const int past = a.tiles_m;   // a sub-tile row outside the tensor
        load_tile<OP, Policy<OP, ROW, COL>::x>(a, l, tm0, tk, wa);
        int g = 0;
        for (; g + 1 < n; g += 2) {
            load_tile<OP, Policy<OP, ROW, COL>::x>(a, l, tm0 + g + 1, tk, wb);
            __builtin_amdgcn_sched_barrier(0);
            tile_step<OP, FMT, ROW, COL, DBIAS, RAG>(a, l, wa, srow, st, tm0 + g, tk, g, n, dsum);
            load_tile<OP, Policy<OP, ROW, COL>::x>(a, l, g + 2 < n ? tm0 + g + 2 : past, tk, wa);
            __builtin_amdgcn_sched_barrier(0);
            tile_step<OP, FMT, ROW, COL, DBIAS, RAG>(a, l, wb, srow, st, tm0 + g + 1, tk, g + 1, n,
                                                    dsum);
        }
        if (g < n)
            tile_step<OP, FMT, ROW, COL, DBIAS, RAG>(a, l, wa, srow, st, tm0 + g, tk, g, n, dsum);
    } else {
        uint32_t w[kRowsPerLane][4];
        for (int g = 0; g < n; g++) {
            if constexpr (OP == OP_DSWIGLU || OP == OP_DGEGLU) {
                // a strip wholly inside one half computes only that half's
                // values (d_linear needs no derivative, d_gate no activation)
                const int64_t k0 = (int64_t)tk * kTileK;
                if (k0 + kTileK <= a.lin_off)
                    load_tile<OP, Policy<OP, ROW, COL>::x, 1>(a, l, tm0 + g, tk, w);
                else if (k0 >= a.lin_off)
                    load_tile<OP, Policy<OP, ROW, COL>::x, 0>(a, l, tm0 + g, tk, w);
                else
                    load_tile<OP, Policy<OP, ROW, COL>::x, 2>(a, l, tm0 + g, tk, w);
            } else {
                load_tile<OP, Policy<OP, ROW, COL>::x>(a, l, tm0 + g, tk, w);
            }
            tile_step<OP, FMT, ROW, COL, DBIAS, RAG>(a, l, w, srow, st, tm0 + g, tk, g, n, dsum);
        }
    }
    if constexpr (COL)
        col_flush_s<Policy<OP, ROW, COL>::s_col>(a, *st, rg, tk, n);

    if constexpr (DBIAS) {
        // per-lane sums (rows in order, sub-tiles in order), then the 8
        // lane-halves of the workgroup in order: one fp32 partial per
        // (strip segment, column)
        // the cross-wave sums reuse the transposed-output stage when there is
        // one (its q part is no longer read), which keeps the LDS of a
        // workgroup small enough for three per CU
        float4 (*red)[kTileK / 4];
        if constexpr (COL) {
            red = reinterpret_cast<float4 (*)[kTileK / 4]>(&st->q[0][0][0]);
        } else {
            __shared__ float4 red_own[2 * kWaves][kTileK / 4];
            red = red_own;
        }
        const int slot = 2 * l.wave + l.half;
        red[slot][l.cl * 2] = make_float4(dsum[0], dsum[1], dsum[2], dsum[3]);
        red[slot][l.cl * 2 + 1] = make_float4(dsum[4], dsum[5], dsum[6], dsum[7]);
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

// The walk (rg) and strip (tk) of this workgroup.  Workgroup ids are
// remapped so that each XCD gets a contiguous run of jobs (xcd_tile), except
// for the dGeGLU cast with halves of whole strips: there the d_gate strips of
// all walks come first and the d_linear strips after them, in dispatch order,
// so that a CU runs one half's code at a time (the two halves take different
// arithmetic; 8192 x 8192 out: 128 -> 126 us, 8-expert grouped: 147 -> 134
// us).  The dSwiGLU cast keeps the XCD order: its d_linear strips re-read the
// gate and grad their d_gate strips have just brought into L2 (half-ordered:
// 123 -> 129 us).
template <int OP>
__device__ __forceinline__ void job_of(const MxArgs &a, int &rg, int &tk)
{
    if constexpr (OP == OP_DGEGLU) {
        if ((a.lin_off & (kTileK - 1)) == 0) {
            const int th = a.tiles_k >> 1, nw = (int)gridDim.x >> 1;
            const int b = (int)blockIdx.x, half = b >= nw ? 1 : 0, r = b - half * nw;
            rg = r / th;
            tk = half * th + (r - rg * th);
            return;
        }
    }
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    rg = job / a.tiles_k;
    tk = job - rg * a.tiles_k;
}

template <int OP, int FMT, bool ROW, bool COL, bool DBIAS>
__global__ __launch_bounds__(kThreads, (min_blocks<OP, DBIAS>())) void mx_cast_kernel(MxArgs a)
{
    int rg, tk;
    job_of<OP>(a, rg, tk);
    mx_cast_walk<OP, FMT, ROW, COL, DBIAS>(a, rg, tk);
}

// Grouped: walk rg (numbered across all groups) belongs to the group g with
// walk0[g] <= rg < walk0[g + 1]; that group is cast as a tensor of its own,
// its inputs and outputs found at the group's offsets.
template <int OP, int FMT, bool ROW, bool COL, bool DBIAS, bool RAG>
__global__ __launch_bounds__(kThreads, (min_blocks<OP, DBIAS, RAG>())) void mx_cast_grouped_kernel(
    MxArgs a, GroupTable gt)
{
    int rg, tk;
    job_of<OP>(a, rg, tk);
    int g = 0;
    while (g + 1 < gt.count && gt.walk0[g + 1] <= rg)
        g++;
    const int64_t r0 = gt.row0[g];
    MxArgs b = a;
    b.M = gt.row0[g + 1] - r0;
    b.x = a.x + r0 * a.ldx;
    b.aux = a.aux ? a.aux + r0 * a.ldg : nullptr;
    b.q_row = a.q_row ? a.q_row + r0 * a.K : nullptr;
    b.s_row = a.s_row ? a.s_row + gt.srow_off[g] : nullptr;
    b.q_col = a.q_col ? a.q_col + a.K * r0 : nullptr;
    b.s_col = a.s_col ? a.s_col + gt.scol_off[g] : nullptr;
    b.partials = a.partials ? a.partials + (int64_t)gt.walk0[g] * a.K : nullptr;
    b.tiles_m = (int)((b.M + kTileM - 1) / kTileM);
    b.group = gt.len[g];
    b.groups_m = gt.walk0[g + 1] - gt.walk0[g];
    mx_cast_walk<OP, FMT, ROW, COL, DBIAS, RAG>(b, rg - gt.walk0[g], tk);
}

template <int OP, int FMT, bool ROW, bool COL, bool DBIAS, bool GROUPED, bool RAG>
hipError_t launch_one(const MxArgs &a, const GroupTable *gt, hipStream_t s)
{
    static_assert(GROUPED || !RAG, "transposed rows at any byte: the grouped kernel only");
    const int blocks = a.groups_m * a.tiles_k;
    if constexpr (GROUPED)
        hipLaunchKernelGGL((mx_cast_grouped_kernel<OP, FMT, ROW, COL, DBIAS, RAG>), dim3(blocks),
                           dim3(kThreads), 0, s, a, *gt);
    else
        hipLaunchKernelGGL((mx_cast_kernel<OP, FMT, ROW, COL, DBIAS>), dim3(blocks),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int OP, int FMT, bool DBIAS, bool GROUPED, bool RAG>
hipError_t launch_axis(unsigned axis, const MxArgs &a, const GroupTable *gt, hipStream_t s)
{
    switch (axis) {
    case 1u:
        // row-wise alone has no transposed rows to align: never the RAG variant
        if constexpr (RAG)
            return hipErrorInvalidValue;
        else
            return launch_one<OP, FMT, true, false, DBIAS, GROUPED, false>(a, gt, s);
    case 2u: return launch_one<OP, FMT, false, true, DBIAS, GROUPED, RAG>(a, gt, s);
    case 3u: return launch_one<OP, FMT, true, true, DBIAS, GROUPED, RAG>(a, gt, s);
    default: return hipErrorInvalidValue;
    }
}

// Every pre-op, output set and dbias choice of one format, plain (gt null)
// or grouped.
template <int FMT, bool GROUPED, bool RAG>
hipError_t launch_mx_cast_fmt(int op, unsigned axis, bool dbias, const MxArgs &a,
                              const GroupTable *gt, hipStream_t s)
{
    switch (op) {
    case OP_PLAIN:
        return dbias ? launch_axis<OP_PLAIN, FMT, true, GROUPED, RAG>(axis, a, gt, s)
                     : launch_axis<OP_PLAIN, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_GELU:
        return dbias ? launch_axis<OP_GELU, FMT, true, GROUPED, RAG>(axis, a, gt, s)
                     : launch_axis<OP_GELU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_DGELU:
        return dbias ? launch_axis<OP_DGELU, FMT, true, GROUPED, RAG>(axis, a, gt, s)
                     : launch_axis<OP_DGELU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_SWIGLU:
        return launch_axis<OP_SWIGLU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_GEGLU:
        return launch_axis<OP_GEGLU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_DSILU:
        return dbias ? launch_axis<OP_DSILU, FMT, true, GROUPED, RAG>(axis, a, gt, s)
                     : launch_axis<OP_DSILU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_DSWIGLU:
        return launch_axis<OP_DSWIGLU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    case OP_DGEGLU:
        return launch_axis<OP_DGEGLU, FMT, false, GROUPED, RAG>(axis, a, gt, s);
    default:
        return hipErrorInvalidValue;
    }
}

// Instantiated once each, in mx_cast_fmt_*.hip (plain), mx_cast_grp_*.hip
// (grouped) and mx_cast_rag_*.hip (grouped, transposed rows at any byte).
#define MXK_DECLARE_FMT(F, G, R)                                                               \
    extern template hipError_t launch_mx_cast_fmt<F, G, R>(int, unsigned, bool, const MxArgs &, \
                                                           const GroupTable *, hipStream_t);
MXK_DECLARE_FMT(0, false, false)
MXK_DECLARE_FMT(kFmtE5M2, false, false)
MXK_DECLARE_FMT(kFmtRoundUp, false, false)
MXK_DECLARE_FMT(kFmtE5M2 | kFmtRoundUp, false, false)
MXK_DECLARE_FMT(0, true, false)
MXK_DECLARE_FMT(kFmtE5M2, true, false)
MXK_DECLARE_FMT(kFmtRoundUp, true, false)
MXK_DECLARE_FMT(kFmtE5M2 | kFmtRoundUp, true, false)
MXK_DECLARE_FMT(0, true, true)
MXK_DECLARE_FMT(kFmtE5M2, true, true)
MXK_DECLARE_FMT(kFmtRoundUp, true, true)
MXK_DECLARE_FMT(kFmtE5M2 | kFmtRoundUp, true, true)
#undef MXK_DECLARE_FMT

}  // namespace mxk
