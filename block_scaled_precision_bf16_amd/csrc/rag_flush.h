// rag_flush.h -- the transposed output of a cast whose transposed rows
// start at any byte (row counts, or the rows before a group, that are not
// multiples of 16), shared by the MXFP8 and NVFP4 tiled kernels.
//
// A workgroup walks down a strip of transposed rows; each step of the walk
// (an MXFP8 sub-tile, an NVFP4 pair of sub-tiles) adds 128 bytes to every
// transposed row, staged in LDS.  Row kr's bytes of a step start at an
// address whose offset sft within its 128-byte line is the same at every
// step of the walk (steps are 128 bytes apart), so a step writes the whole
// line that starts sft bytes before its first byte: the previous step's last
// sft bytes (still in the other of two staged tiles) and its own first
// 128 - sft, as 8 aligned 16-byte pieces.  Its own last sft bytes go out with
// the next step.  Only bytes of the walk are written: at its first step the
// sft bytes before it belong to the walk or group before, and its last step
// also writes the line after, up to the row's end (rem bytes of the step);
// the pieces holding other bytes as well -- at most one at each end of a row
// -- leave in naturally aligned stores of 1, 2, 4 and 8 bytes, at those two
// steps only.  Thread t writes piece t % 8 of rows t / 8 + 32 i (and of the
// line after), and the end pieces of row t.
//
// A staged view V gives, for transposed row kr, V::chunk(kr, c): the
// previous step's 16-byte chunk c (c < 8), the current step's chunk c - 8
// (8 <= c < 16), any value beyond.
#pragma once

#include <type_traits>

#include "bufio.h"
#include "launch.h"

namespace mxk {

// Bytes s .. s + 15 (0 <= s < 16) of the 32 bytes p (bytes 0-15) and c
// (bytes 16-31): the dword shift in two rounds of selects, then the byte
// shift.  Written on named words, not an array: the compiler turns selects
// among an array's elements into an indexed load from scratch memory.
__device__ __forceinline__ uint4 window16(uint4 p, uint4 c, uint32_t s)
{
    const bool d1 = (s & 4u) != 0, d2 = (s & 8u) != 0;
    const uint32_t y0 = d1 ? p.y : p.x, y1 = d1 ? p.z : p.y, y2 = d1 ? p.w : p.z;
    const uint32_t y3 = d1 ? c.x : p.w, y4 = d1 ? c.y : c.x, y5 = d1 ? c.z : c.y;
    const uint32_t y6 = d1 ? c.w : c.z;
    const uint32_t x0 = d2 ? y2 : y0, x1 = d2 ? y3 : y1, x2 = d2 ? y4 : y2;
    const uint32_t x3 = d2 ? y5 : y3, x4 = d2 ? y6 : y4;
    const uint32_t sh = s & 3u;
    return make_uint4(__builtin_amdgcn_alignbyte(x1, x0, sh), __builtin_amdgcn_alignbyte(x2, x1, sh),
                      __builtin_amdgcn_alignbyte(x3, x2, sh), __builtin_amdgcn_alignbyte(x4, x3, sh));
}

// The 16 bytes at position u (0 <= u < 384) of row kr in V's sequence.
template <class V>
__device__ __forceinline__ uint4 rag_bytes(const V &v, int kr, int u)
{
    const int c = u >> 4;
    return window16(v.chunk(kr, c), v.chunk(kr, c + 1), (uint32_t)(u & 15));
}

// Bytes b .. b + S - 1 of the 16 bytes w (b a multiple of S) to offset off.
template <int S>
__device__ __forceinline__ void rag_store_at(rsrc_t rc, uint32_t off, uint4 w, int b)
{
    if constexpr (S == 8) {
        const bool hi = (b & 8) != 0;
        buf_store8(rc, off, make_uint2(hi ? w.z : w.x, hi ? w.w : w.y));
    } else {
        const uint32_t lo = (b & 4) ? w.y : w.x, up = (b & 4) ? w.w : w.z;
        const uint32_t d = (b & 8) ? up : lo;
        if constexpr (S == 4)
            buf_store4(rc, off, d);
        else if constexpr (S == 2)
            buf_store2(rc, off, (uint16_t)(d >> (8 * (b & 2))));
        else
            buf_store1(rc, off, (uint8_t)(d >> (8 * (b & 3))));
    }
}

// Bytes b0 .. b1 - 1 (0 <= b0 < b1 <= 16, less than the whole piece: the
// end pieces are partial) of the 16 bytes w to the 16-byte aligned offset pa (lanes with `on` false store nothing), in naturally
// aligned stores: upwards by size while b0's low bits are set (UP; b0 = 0
// needs none of them), then downwards by size.  Once a size does not fit
// upwards, no larger one does, so the downward stores start at a multiple of
// that size and stay aligned.
template <bool UP>
__device__ __forceinline__ void rag_store_range(rsrc_t rc, bool on, uint32_t pa, uint4 w, int b0, int b1)
{
    int b = b0;
    const auto put = [&](auto size, bool go) {
        constexpr int S = decltype(size)::value;
        go = go && on && b + S <= b1;
        rag_store_at<S>(rc, go ? pa + (uint32_t)b : kDead, w, b);
        b += go ? S : 0;
    };
    if (UP) {
        put(std::integral_constant<int, 1>{}, (b & 1) != 0);
        put(std::integral_constant<int, 2>{}, (b & 2) != 0);
        put(std::integral_constant<int, 4>{}, (b & 4) != 0);
        put(std::integral_constant<int, 8>{}, (b & 8) != 0);
    }
    put(std::integral_constant<int, 8>{}, true);
    put(std::integral_constant<int, 4>{}, true);
    put(std::integral_constant<int, 2>{}, true);
    put(std::integral_constant<int, 1>{}, true);
}

// One step of the walk: rc covers the transposed output from the line
// boundary at or below the step's first byte of the strip's first row
// (base = that byte's offset from the boundary); transposed rows are pitch
// bytes apart, rows at or past `rows` (counted from the strip's first) do not
// exist; the step holds rem <= 128 bytes of each row.
template <int AUX, class V>
__device__ __forceinline__ void rag_flush_lines(const V &v, rsrc_t rc, uint32_t base, uint32_t pitch,
                                                int64_t rows, int rem, bool first, bool last)
{
    const int t = (int)threadIdx.x;
    const int j = t & 7;
    // the rows' offsets are the same at every step; kept opaque here, they
    // are formed again each time instead of being held across the walk
    asm volatile("" : "+v"(base));
    // bytes lo .. rem - 1 of the step's row segment are its to write
    // (negative: the previous step's)
    const int lo = first ? 0 : -128;
    const int nr = rows < 256 ? (int)rows : 256;   // rows of the strip that exist
    // two rows' pieces in flight at a time: enough to overlap the reads, and
    // the registers stay within what the casts around it leave
#pragma unroll 2
    for (int i = 0; i < 256 / 32; i++) {
        const int kr = (t >> 3) + 32 * i;
        const uint32_t at = base + (uint32_t)kr * pitch;  // the row's first byte of the step
        const int sft = (int)(at & 127u);
        const int p0 = 16 * j - sft;                       // the piece's first byte in the segment
        const uint4 w = rag_bytes(v, kr, p0 + 128);
        const bool whole = kr < nr && p0 >= lo && p0 + 16 <= rem;
        buf_store16<AUX>(rc, whole ? at - (uint32_t)sft + 16u * j : kDead, w);
    }
    if (last) {
        // the line after, whole pieces (the same lanes per row)
#pragma unroll 2
        for (int i = 0; i < 256 / 32; i++) {
            const int kr = (t >> 3) + 32 * i;
            const uint32_t at = base + (uint32_t)kr * pitch;
            const int sft = (int)(at & 127u);
            const int p0 = 128 + 16 * j - sft;
            const bool whole = kr < nr && p0 + 16 <= rem;
            buf_store16<AUX>(rc, whole ? at - (uint32_t)sft + (uint32_t)(128 + 16 * j) : kDead,
                             rag_bytes(v, kr, p0 + 128));
        }
    }
    if (!(first || last))
        return;
    // the end pieces, one row per thread: at the first step the walk's bytes
    // of the piece that holds the row's first byte (if the piece starts
    // before it), at the last those of the piece that holds its last byte (if
    // it ends after it)
    const int kr = t;
    const uint32_t at = base + (uint32_t)kr * pitch;
    const int sft = (int)(at & 127u);
    const int o = sft & 15, et = (rem + sft) & 15;
    const int qh = sft >> 4, qt = (rem - 1 + sft) >> 4;
    const bool head = kr < nr && first && o != 0;
    // a walk of one step whose bytes all lie in the head piece has no tail
    const bool tail = kr < nr && last && et != 0 && !(head && qt == qh);
    if (__builtin_amdgcn_ballot_w64(head) != 0)
        rag_store_range<true>(rc, head, at - (uint32_t)sft + 16u * qh,
                              rag_bytes(v, kr, 128 - o), o, min(16, o + rem));
    if (__builtin_amdgcn_ballot_w64(tail) != 0)
        rag_store_range<false>(rc, tail, at - (uint32_t)sft + 16u * qt,
                               rag_bytes(v, kr, 16 * qt - sft + 128), 0, et);
}

}  // namespace mxk
