// any_common.h -- pieces shared by the casts of any shape (mx_cast_any.hip
// for MXFP8, nvfp4_any.hip for NVFP4): rows that start at any byte.
//
// Both kernels walk a 128-column strip in steps of 64 rows.  Each thread
// loads one column of 32 rows with 2-byte loads through one scalar
// descriptor per 32 rows; the codes of a step leave through LDS:
//   * row-wise, each row's segment of the step (128 or 64 bytes) as the
//     aligned dwords inside it plus at most 3 head and 3 tail bytes, or as
//     16-byte pieces when every row starts 16-byte aligned (flush_rows);
//   * transposed, each transposed row's bytes of the step (64 or 32) start
//     at the same offset within a chunk of that size at every step, so a
//     two-step ring in LDS lets every step write whole aligned chunks as
//     16-byte pieces; only a walk's first and last chunks leave in narrower
//     stores (flush_cols).
#pragma once

#include "bufio.h"
#include "device_math.h"
#include "launch.h"
#include "rag_flush.h"

namespace mxk {

template <int AUX = 0>
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, AUX);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Low bits of the absolute byte address p + off.
__device__ __forceinline__ uint32_t addr_low(const void *p, int64_t off, uint32_t mask)
{
    return (uint32_t)((reinterpret_cast<uintptr_t>(p) + (uint64_t)off) & mask);
}

// The four bytes at staged position i (any alignment) of an LDS row whose
// dwords at i & ~3 and (i & ~3) + 4 exist.
__device__ __forceinline__ uint32_t lds_word_at(const uint8_t *row, int i)
{
    const uint32_t *w = reinterpret_cast<const uint32_t *>(row + (i & ~3));
    return __builtin_amdgcn_alignbyte(w[1], w[0], (uint32_t)(i & 3));
}

// Descriptor of a bf16 tensor p[rows][ld] from row `row`, column `col` to
// the tensor's end (size 0 for a row at or past the last).
__device__ __forceinline__ rsrc_t row_rsrc(const uint16_t *p, int64_t row, int64_t ld, int64_t rows,
                                           int64_t col = 0)
{
    return make_rsrc(p, 2 * (row * ld + col), 2 * rows * ld);
}

// Rows m .. m + 31 of a bf16 tensor p[rows][ld] seen from column col: one
// scalar descriptor from row m, column col to the tensor's end, row i at byte
// i * pitch of it.  A lane adds its column's offset.  Row i past the last
// starts at or past the descriptor's end, so only columns need a mask: with
// ld <= 2^23, every offset of rows 0 .. 31 is below 2^30 and kDead plus any
// of them stays below 2^32.  (Where 2 (rows - m) ld exceeds the largest
// descriptor, all 32 rows exist.)
struct Rows32 {
    rsrc_t r;
    uint32_t pitch;
};

__device__ __forceinline__ Rows32 rows32(const uint16_t *p, int64_t m, int64_t ld, int64_t rows,
                                         int64_t col = 0)
{
    return Rows32{row_rsrc(p, m, ld, rows, col), (uint32_t)(2 * ld)};
}

__device__ __forceinline__ uint32_t load_row(const Rows32 &v, int i, uint32_t off)
{
    return buf_load2(v.r, off + (uint32_t)i * v.pitch);
}

// A lane's column offset, opaque to the compiler for one step: its 32 row
// offsets are then formed at each step (one add per load) instead of being
// held in registers across the whole walk.
__device__ __forceinline__ uint32_t step_offset(uint32_t off)
{
    asm volatile("" : "+v"(off));
    return off;
}

// Raw bf16 of column k, rows m .. m + 31 of x[rows][ld] (0 past the last row
// or when col_ok is false): word i holds rows 2i (low half) and 2i + 1.
__device__ __forceinline__ void load_column32(const uint16_t *x, int64_t ld, int64_t rows,
                                              int64_t m, int64_t k, bool col_ok, uint32_t (&w)[16])
{
    const Rows32 v = rows32(x, m, ld, rows);
    const uint32_t ox = step_offset(col_ok ? (uint32_t)(2 * k) : kDead);
    uint32_t e[32];
#pragma unroll
    for (int i = 0; i < 32; i++)
        e[i] = load_row(v, i, ox);
#pragma unroll
    for (int i = 0; i < 16; i++)
        w[i] = pack2(e[2 * i], e[2 * i + 1]);
}

// Staged row-wise codes of a step -> out: rows row0 .. row0 + rows_left - 1
// (at most 64), each a segment of seg <= SEG bytes starting at byte
// (row0 + r) * stride + col0 of out (total bytes), staged at
// stage + r * sstride (rows of SEG + 4 readable bytes).  Rows whose bytes
// start 16-byte aligned (out + col0 and stride aligned) leave as 16-byte
// pieces; otherwise each row leaves as the aligned dwords inside its segment,
// each assembled from two aligned LDS dwords, plus at most 3 head and 3 tail
// bytes.  Every instruction's rows are the same for all lanes of a group; the
// descriptor starts at row row0, so rows past the tensor lie outside it.
template <int SEG>
__device__ __forceinline__ void flush_rows(uint8_t *out, int64_t stride, int64_t row0, int64_t col0,
                                           int64_t total, int rows_left, int seg,
                                           const uint8_t *stage, int sstride)
{
    static_assert(SEG == 128 || SEG == 64, "segments of 128 or 64 bytes");
    const int lane = (int)threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const rsrc_t rq = make_rsrc(out, row0 * stride + col0, total);
    if ((stride & 15) == 0 && addr_low(out, col0, 15) == 0) {
        constexpr int per = SEG / 16;               // 16-byte pieces per row
        constexpr int rows_per = 64 / per;          // rows per wave instruction
        const int sub = lane / per, p = lane % per;
#pragma unroll
        for (int i = 0; i < kAnyTileM / (4 * rows_per); i++) {
            const int r = rows_per * (wv + 4 * i) + sub;
            const bool ok = r < rows_left && 16 * p < seg;
            buf_store16(rq, ok ? (uint32_t)(r * stride + 16 * p) : kDead,
                        *reinterpret_cast<const uint4 *>(stage + r * sstride + 16 * p));
        }
        return;
    }
    // aligned dwords: SEG / 4 lanes per row
    constexpr int per = SEG / 4;
    constexpr int rows_per = 64 / per;
#pragma unroll
    for (int i = 0; i < kAnyTileM / (4 * rows_per); i++) {
        const int r = rows_per * (wv + 4 * i) + lane / per, u = lane % per;
        const uint32_t al = addr_low(out, (row0 + r) * stride + col0, 3);
        const int head = min(seg, (int)((4 - al) & 3));
        const int nd = (seg - head) >> 2;
        const int i0 = head + 4 * u;
        const bool ok = r < rows_left && u < nd;
        buf_store4(rq, ok ? (uint32_t)(r * stride + i0) : kDead,
                   lds_word_at(stage + r * sstride, ok ? i0 : 0));
    }
    // head bytes (slots 0-2) and tail bytes (slots 3-5) of 8 rows per instruction
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = 8 * (wv + 4 * i) + (lane >> 3), slot = lane & 7;
        const uint32_t al = addr_low(out, (row0 + r) * stride + col0, 3);
        const int head = min(seg, (int)((4 - al) & 3));
        const int tail0 = head + 4 * ((seg - head) >> 2);
        const int b = slot < 3 ? slot : tail0 + slot - 3;
        const bool ok = r < rows_left && (slot < 3 ? slot < head : slot < 6 && b < seg);
        buf_store1(rq, ok ? (uint32_t)(r * stride + b) : kDead, stage[r * sstride + (ok ? b : 0)]);
    }
}

// Transposed codes of step s -> out (transposed rows k0 .. k0 + 127 of K,
// tstride bytes apart; this step's bytes start at byte pos of each and hold
// rem <= CH bytes).  Transposed row c's bytes of the step start at an
// address whose offset within its CH-byte chunk, sft, is the same at every
// step (steps are CH bytes apart).  The step writes the chunk that starts sft
// bytes before its first byte: bytes 0 .. sft - 1 are the previous step's
// last bytes, still in the other half of the ring (ring + c * rstride, step s
// at bytes CH (s % 2) .. CH (s % 2) + CH - 1), and bytes sft .. CH - 1 this
// step's first.  Its last sft bytes wait for the next step; the walk's last
// step writes them too.  At the walk's first step the chunk's first sft
// bytes belong to the walk before and are left alone.  Whole 16-byte pieces
// leave as 16-byte stores assembled from aligned LDS dwords; of the pieces
// with bytes outside the walk, the walk's bytes leave in naturally aligned
// stores of 1, 2, 4 and 8 bytes.
template <int CH>
__device__ __forceinline__ void flush_cols(uint8_t *out, int64_t tstride, int64_t k0, int64_t K,
                                           int64_t pos, int rem, int s, bool last,
                                           const uint8_t *ring, int rstride)
{
    static_assert(CH == 64 || CH == 32, "chunks of 64 or 32 bytes");
    constexpr int lg = CH == 64 ? 2 : 1;             // log2 of 16-byte pieces per chunk
    const int t = (int)threadIdx.x;
    const rsrc_t rc = make_rsrc(out, k0 * tstride, K * tstride);
    const int lnp = last ? lg + 1 : lg;             // pieces per transposed row: 2^lnp
    const int np = 1 << lnp;
    for (int i = 0; i < (kAnyTileK * np) / kThreads; i++) {
        const int idx = t + kThreads * i;
        const int c = idx >> lnp, j = idx & (np - 1);
        const int sft = (int)addr_low(out, (k0 + c) * tstride + pos, CH - 1);
        const int lo = s > 0 ? 0 : sft;           // chunk bytes [lo, hi) exist
        const int hi = sft + rem;
        const int64_t co = (int64_t)c * tstride + pos - sft;   // chunk start (< 0 only where lo > 0)
        const int v0 = (CH * (s & 1) - sft + 16 * j) & (2 * CH - 1);   // ring position of byte 16 j
        const uint8_t *rr = ring + c * rstride;
        const bool row_ok = k0 + c < K;
        const bool whole = row_ok && lo <= 16 * j && 16 * j + 16 <= hi;
        uint4 o;
        {
            const uint32_t *w = reinterpret_cast<const uint32_t *>(rr);
            const int f = v0 >> 2, sh = v0 & 3;
            uint32_t d[5];
#pragma unroll
            for (int e = 0; e < 5; e++)
                d[e] = w[(f + e) & (CH / 2 - 1)];
            o = make_uint4(__builtin_amdgcn_alignbyte(d[1], d[0], sh),
                           __builtin_amdgcn_alignbyte(d[2], d[1], sh),
                           __builtin_amdgcn_alignbyte(d[3], d[2], sh),
                           __builtin_amdgcn_alignbyte(d[4], d[3], sh));
        }
        buf_store16(rc, whole ? (uint32_t)(co + 16 * j) : kDead, o);
        const bool part = row_ok && !whole && 16 * j < hi && 16 * j + 16 > lo;
        if (__builtin_amdgcn_ballot_w64(part) != 0)   // uniform: first and last steps only
            rag_store_range<true>(rc, part, (uint32_t)(co + 16 * j), o,
                                  lo > 16 * j ? lo - 16 * j : 0, hi < 16 * j + 16 ? hi - 16 * j : 16);
    }
}

}  // namespace mxk
