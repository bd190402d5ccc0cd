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

template <int AUX = 0>
__device__ __forceinline__ void buf_store2(rsrc_t r, uint32_t off, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, AUX);
}

template <int AUX, int CH, int W>
__device__ __forceinline__ void flush_scale_rows_ch(rsrc_t rs, const uint8_t (&s)[kTileK][W],
                                                    int64_t k0, int64_t K, int64_t pitch,
                                                    int count)
{
    const int t = (int)threadIdx.x;
    const int pieces = count / CH;                        // per row
    for (int i = 0; i < pieces; i++) {
        const int idx = t + kThreads * i;                 // (row, piece) pair
        const int c = idx / pieces, q = idx - c * pieces;
        const uint32_t off = k0 + c < K ? (uint32_t)(c * pitch) + CH * q : kDead;
        const uint8_t *src = &s[c][CH * q];
        if constexpr (CH == 16)
            buf_store16<AUX>(rs, off, *reinterpret_cast<const uint4 *>(src));
        else if constexpr (CH == 8)
            buf_store8<AUX>(rs, off, *reinterpret_cast<const uint2 *>(src));
        else if constexpr (CH == 4)
            buf_store4<AUX>(rs, off, *reinterpret_cast<const uint32_t *>(src));
        else if constexpr (CH == 2)
            buf_store2<AUX>(rs, off, *reinterpret_cast<const uint16_t *>(src));
        else
            buf_store1<AUX>(rs, off, *src);
    }
}

// rs covers the scale tensor from byte k0 * pitch + first of `base`; rows at
// or beyond K are skipped.  count <= W.
template <int AUX, int W>
__device__ __forceinline__ void flush_scale_rows(rsrc_t rs, const uint8_t (&s)[kTileK][W],
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
