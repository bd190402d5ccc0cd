// mx_cast.hip -- the helper kernels of the MXFP8 casts (the dbias reduction
// over strip segments and the fused-value kernel that exposes each pre-op's
// bf16 result) and the dispatch of the cast kernel to its format's
// instantiation.

#include "mx_cast.h"

#include <mutex>

namespace mxk {

// The dbias partials of mx_quantize_noalloc, for callers that cannot
// allocate: one copy per GPU, alive until the process ends.  In host code
// the name stands for a host-side shadow, not the device array, so kernels
// only ever get the address that noalloc_scratch looks up.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(hipStream_t s, float **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // the lookup runs with the stream's device current
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess)
                e = back;
        }
        if (e != hipSuccess)
            return e;
        addr[dev] = static_cast<float *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
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

// dbias[g][k] = sum over group g's walks (in order) of partials[walk][k];
// 0 for a group without rows.  Grid: (ceil(K / 256), groups).
__global__ __launch_bounds__(256) void dbias_reduce_grouped_kernel(const float *partials,
                                                                   GroupTable gt, int64_t K,
                                                                   float *dbias)
{
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int g = (int)blockIdx.y;
    if (k >= K)
        return;
    float acc = 0.0f;
    for (int t = gt.walk0[g]; t < gt.walk0[g + 1]; t++)
        acc += partials[(int64_t)t * K + k];
    dbias[(int64_t)g * K + k] = acc;
}

// y = fused value of each element; 8 elements per thread.  Gated ops read
// the row [gate | linear] of width 2K; the gated backward ops read that row
// and grad[M][K] and write the row [d_gate | d_linear] of y[M][2K].
template <int OP>
__global__ __launch_bounds__(256) void fused_values_kernel(const uint16_t *x, const uint16_t *aux,
                                                           int64_t M, int64_t K, uint16_t *y)
{
    constexpr bool dgated = OP == OP_DSWIGLU || OP == OP_DGEGLU;
    const int64_t W = dgated ? 2 * K : K;                  // width of y
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= M * W)
        return;
    const int64_t row = i / W, col = i - row * W;
    uint4 o;
    if constexpr (dgated) {
        const bool gate_half = col < K;
        const int64_t n = gate_half ? col : col - K;
        const uint4 g = *reinterpret_cast<const uint4 *>(x + row * 2 * K + n);
        const uint4 dy = *reinterpret_cast<const uint4 *>(aux + row * K + n);
        const uint4 li = *reinterpret_cast<const uint4 *>(x + row * 2 * K + K + n);
        o.x = dgated_pair<OP>(g.x, dy.x, li.x, gate_half);
        o.y = dgated_pair<OP>(g.y, dy.y, li.y, gate_half);
        o.z = dgated_pair<OP>(g.z, dy.z, li.z, gate_half);
        o.w = dgated_pair<OP>(g.w, dy.w, li.w, gate_half);
    } else {
        const bool gated = OP == OP_SWIGLU || OP == OP_GEGLU;
        const uint16_t *pa = gated ? x + row * 2 * K + col : x + i;
        const uint16_t *pb = gated ? pa + K : aux + i;
        const uint4 va = *reinterpret_cast<const uint4 *>(pa);
        const uint4 vb = *reinterpret_cast<const uint4 *>(pb);
        o.x = fused_pair<OP>(va.x, vb.x);
        o.y = fused_pair<OP>(va.y, vb.y);
        o.z = fused_pair<OP>(va.z, vb.z);
        o.w = fused_pair<OP>(va.w, vb.w);
    }
    *reinterpret_cast<uint4 *>(y + i) = o;
}

template <bool GROUPED, bool RAG>
static hipError_t dispatch_fmt(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                               const GroupTable *gt, hipStream_t s)
{
    switch (fmt) {
    case 0u: return launch_mx_cast_fmt<0, GROUPED, RAG>(op, axis, dbias, a, gt, s);
    case kFmtE5M2: return launch_mx_cast_fmt<kFmtE5M2, GROUPED, RAG>(op, axis, dbias, a, gt, s);
    case kFmtRoundUp: return launch_mx_cast_fmt<kFmtRoundUp, GROUPED, RAG>(op, axis, dbias, a, gt, s);
    case kFmtE5M2 | kFmtRoundUp:
        return launch_mx_cast_fmt<kFmtE5M2 | kFmtRoundUp, GROUPED, RAG>(op, axis, dbias, a, gt, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mx_cast(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                          hipStream_t s)
{
    return dispatch_fmt<false, false>(op, axis, fmt, dbias, a, nullptr, s);
}

hipError_t launch_mx_cast_grouped(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                                  const GroupTable &gt, hipStream_t s)
{
    return dispatch_fmt<true, false>(op, axis, fmt, dbias, a, &gt, s);
}

hipError_t launch_mx_cast_ragged(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                                 const GroupTable &gt, hipStream_t s)
{
    return dispatch_fmt<true, true>(op, axis, fmt, dbias, a, &gt, s);
}

hipError_t launch_dbias_reduce(const float *partials, int segments, int64_t K, float *dbias,
                               hipStream_t s)
{
    const int64_t blocks = (K + 255) / 256;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partials,
                       segments, K, dbias);
    return hipGetLastError();
}

hipError_t launch_dbias_reduce_grouped(const float *partials, const GroupTable &gt, int64_t K,
                                       float *dbias, hipStream_t s)
{
    const dim3 grid((unsigned)((K + 255) / 256), (unsigned)gt.count);
    hipLaunchKernelGGL(dbias_reduce_grouped_kernel, grid, dim3(256), 0, s, partials, gt, K, dbias);
    return hipGetLastError();
}

hipError_t launch_fused_values(int op, const uint16_t *x, const uint16_t *aux, int64_t M,
                               int64_t K, uint16_t *y, hipStream_t s)
{
    const int64_t threads = M * K * (op == OP_DSWIGLU || op == OP_DGEGLU ? 2 : 1) / 8;
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
    case OP_DSILU:
        hipLaunchKernelGGL(fused_values_kernel<OP_DSILU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    case OP_DSWIGLU:
        hipLaunchKernelGGL(fused_values_kernel<OP_DSWIGLU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    case OP_DGEGLU:
        hipLaunchKernelGGL(fused_values_kernel<OP_DGEGLU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mxk
