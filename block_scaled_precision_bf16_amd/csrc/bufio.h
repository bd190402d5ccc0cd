// bufio.h -- raw buffer-resource access for the cast kernels (gfx950).
//
// Every global load and store of the cast kernels goes through a buffer
// resource (a 128-bit descriptor: base address, size in bytes) with a 32-bit
// per-lane byte offset.  An offset at or beyond the size is out of range: the
// hardware returns 0 for such a load and drops such a store, without touching
// memory.  Lanes, waves or whole sub-tiles that lie outside the tensor are
// therefore masked by giving them the offset kDead (or a descriptor of size 0)
// instead of branching around the instruction.  This keeps the number of
// memory instructions the same on every path through a kernel, which lets the
// compiler's wait-counter bookkeeping stay exact: a load issued for the next
// sub-tile is then not waited for while the current one is converted.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

using rsrc_t = __amdgpu_buffer_rsrc_t;

// Word 3 of a gfx9 raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
// Descriptors never cover more than 2^31 - 1 bytes, so kDead is always out
// of range; callers keep every live offset below 2^31.
constexpr int64_t kMaxRecords = 0x7FFFFFFF;
constexpr uint32_t kDead = 0x80000000u;

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Descriptor for the bytes [offset, total) of the allocation at base; size 0
// (every access out of range) when offset >= total.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t offset, int64_t total)
{
    const int64_t left = total - offset;
    const char *p = static_cast<const char *>(base) + (left > 0 ? offset : 0);
    const int n = (int)(left <= 0 ? 0 : (left > kMaxRecords ? kMaxRecords : left));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, n, kRsrcWord3);
}

// AUX is the instruction's cache-policy operand: 0 for the default policy,
// kNT for the non-temporal (streaming) hint, kSC1 for the device-scope
// coherence bit (SC1) of CDNA3/CDNA4 memory instructions.
constexpr int kNT = 2;
constexpr int kSC1 = 16;

template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int AUX = 0>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, uint4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)off, 0, AUX);
}

template <int AUX = 0>
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, (int)off, 0, AUX);
}

template <int AUX = 0>
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, AUX);
}

template <int AUX = 0>
__device__ __forceinline__ void buf_store2(rsrc_t r, uint32_t off, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, AUX);
}

template <int AUX = 0>
__device__ __forceinline__ void buf_store1(rsrc_t r, uint32_t off, uint8_t v)
{
    __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)off, 0, AUX);
}

}  // namespace mxk
