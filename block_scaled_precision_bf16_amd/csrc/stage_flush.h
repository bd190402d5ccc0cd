// stage_flush.h -- writing LDS-staged scale rows out to a row-major scale
// tensor, in the widest pieces the tensor's layout allows (gfx950).
//
// Both cast kernels stage, for the 256 transposed rows of a strip, the
// column-block scales of a whole walk, and write them at its end: row c's
// `count` bytes go to bytes [c * pitch + first, + count) of the scale tensor.
// The pieces of one row go to neighbouring threads, so one store instruction
// touches few cache lines.  Pieces narrower than 16 bytes (rows whose length
// or start is not a multiple of 16) complete their lines only together with
// the neighbouring walks' pieces, so they keep the default cache policy:
// streamed out one by one, they would reach memory as partial-line writes.
#pragma once

#include "bufio.h"
#include "launch.h"

namespace mxk {

// Column-block scales are staged transposed: s[b][pos] holds the scale of
// block b of the walk (a 32-row block of MXFP8, a 16-row block of NVFP4) of
// transposed row kl, at byte pos = kl ^ scol_swz(b).  A lane's 8 columns
// (kl = 8 cl .. 8 cl + 7) are 8 contiguous bytes, so the lane writes its
// scales of one block with one 8-byte store and a half-wave covers a whole
// 256-byte row: no two of its lanes share an LDS bank.  The XOR (bits 4-5 of
// kl, from bits 4-5 of b) spreads the flush's reads of the 16 blocks of one
// 16-byte piece over distinct banks as well.
__device__ __forceinline__ int scol_pos(int b, int kl) { return kl ^ (16 * ((b >> 4) & 3)); }

template <int W>
__device__ __forceinline__ void stage_scales8(uint8_t (&s)[W][kTileK], int b, int cl, uint2 v)
{
    *reinterpret_cast<uint2 *>(&s[b][scol_pos(b, 8 * cl)]) = v;
}

// Eight scale bytes (byte j = value j, j = 0..7) packed for stage_scales8.
__device__ __forceinline__ uint2 pack8(const uint32_t (&b)[8])
{
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                      b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

// Bytes b0 .. b0 + N - 1 of staged transposed row kl, byte i = block b0 + i.
template <int N, int W>
__device__ __forceinline__ void staged_bytes(const uint8_t (&s)[W][kTileK], int b0, int kl,
                                             uint32_t (&w)[(N + 3) / 4])
{
#pragma unroll
    for (int i = 0; i < (N + 3) / 4; i++)
        w[i] = 0;
#pragma unroll
    for (int j = 0; j < N; j++)
        w[j >> 2] |= (uint32_t)s[b0 + j][scol_pos(b0 + j, kl)] << (8 * (j & 3));
}

template <int AUX, int CH, int W>
__device__ __forceinline__ void flush_scale_rows_ch(rsrc_t rs, const uint8_t (&s)[W][kTileK],
                                                    int64_t k0, int64_t K, int64_t pitch,
                                                    int count)
{
    const int t = (int)threadIdx.x;
    const int pieces = count / CH;                        // per row
    for (int i = 0; i < pieces; i++) {
        const int idx = t + kThreads * i;                 // (row, piece) pair
        const int c = idx / pieces, q = idx - c * pieces;
        const uint32_t off = k0 + c < K ? (uint32_t)(c * pitch) + CH * q : kDead;
        uint32_t w[(CH + 3) / 4];
        staged_bytes<CH>(s, CH * q, c, w);
        if constexpr (CH == 16)
            buf_store16<AUX>(rs, off, make_uint4(w[0], w[1], w[2], w[3]));
        else if constexpr (CH == 8)
            buf_store8<AUX>(rs, off, make_uint2(w[0], w[1]));
        else if constexpr (CH == 4)
            buf_store4<AUX>(rs, off, w[0]);
        else if constexpr (CH == 2)
            buf_store2<AUX>(rs, off, (uint16_t)w[0]);
        else
            buf_store1<AUX>(rs, off, (uint8_t)w[0]);
    }
}

// rs covers the scale tensor from byte k0 * pitch + first of `base`; rows at
// or beyond K are skipped.  count <= W; s is the transposed stage above.
template <int AUX, int W>
__device__ __forceinline__ void flush_scale_rows(rsrc_t rs, const uint8_t (&s)[W][kTileK],
                                                 int64_t k0, int64_t K, int64_t pitch,
                                                 int64_t first, int count, const void *base)
{
    const int64_t align = pitch | first | count | (int64_t)(reinterpret_cast<uintptr_t>(base) & 15);
    if ((align & 15) == 0)
        flush_scale_rows_ch<AUX, 16>(rs, s, k0, K, pitch, count);
    else if ((align & 7) == 0)
        flush_scale_rows_ch<0, 8>(rs, s, k0, K, pitch, count);
    else if ((align & 3) == 0)
        flush_scale_rows_ch<0, 4>(rs, s, k0, K, pitch, count);
    else if ((align & 1) == 0)
        flush_scale_rows_ch<0, 2>(rs, s, k0, K, pitch, count);
    else
        flush_scale_rows_ch<0, 1>(rs, s, k0, K, pitch, count);
}

}  // namespace mxk
