// Stand-ins for the kernel launchers of libmxcast (csrc/launch.h) in a
// host-only build of the entry points (csrc/api.cpp): each records that it
// was called and with what, and launches nothing.  Lets the validation and
// launch-planning code run under AddressSanitizer and UBSan on a machine
// without a GPU.
#include "launch_record.h"

namespace mxk {

Record g_rec;

static hipError_t note(int kind)
{
    g_rec.calls++;
    g_rec.kind = kind;
    return hipSuccess;
}

hipError_t launch_mx_cast(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                          hipStream_t)
{
    g_rec.op = op, g_rec.axis = axis, g_rec.fmt = fmt, g_rec.dbias = dbias, g_rec.mx = a;
    return note(kLaunchMx);
}

hipError_t launch_mx_cast_grouped(int op, unsigned axis, unsigned fmt, bool dbias,
                                  const MxArgs &a, const GroupTable &gt, hipStream_t)
{
    g_rec.op = op, g_rec.axis = axis, g_rec.fmt = fmt, g_rec.dbias = dbias, g_rec.mx = a;
    g_rec.gt = gt;
    return note(kLaunchMxGrouped);
}

hipError_t launch_mx_cast_ragged(int op, unsigned axis, unsigned fmt, bool dbias,
                                 const MxArgs &a, const GroupTable &gt, hipStream_t)
{
    g_rec.op = op, g_rec.axis = axis, g_rec.fmt = fmt, g_rec.dbias = dbias, g_rec.mx = a;
    g_rec.gt = gt;
    return note(kLaunchMxRagged);
}

hipError_t launch_mx_cast_any(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                              const GroupTable &gt, hipStream_t)
{
    g_rec.op = op, g_rec.axis = axis, g_rec.fmt = fmt, g_rec.dbias = dbias, g_rec.mx = a;
    g_rec.gt = gt;
    return note(kLaunchMxAny);
}

hipError_t launch_dbias_reduce_grouped(const float *, const GroupTable &gt, int64_t K, float *,
                                       hipStream_t)
{
    g_rec.gt = gt, g_rec.K = K;
    g_rec.reduces++;
    return hipSuccess;
}

hipError_t launch_dbias_reduce(const float *, int segments, int64_t K, float *, hipStream_t)
{
    g_rec.segments = segments, g_rec.K = K;
    g_rec.reduces++;
    return hipSuccess;
}

static float g_fake_scratch[1];

hipError_t noalloc_scratch(hipStream_t, float **ptr)
{
    *ptr = g_fake_scratch;
    return hipSuccess;
}

hipError_t launch_fused_values(int op, const uint16_t *, const uint16_t *, int64_t M, int64_t K,
                               uint16_t *, hipStream_t)
{
    g_rec.op = op, g_rec.M = M, g_rec.K = K;
    return note(kLaunchValues);
}

hipError_t launch_fused_values_any(int op, const uint16_t *, const uint16_t *, int64_t M,
                                   int64_t K, uint16_t *, hipStream_t)
{
    g_rec.op = op, g_rec.M = M, g_rec.K = K;
    return note(kLaunchValuesAny);
}

hipError_t launch_absmax(const uint16_t *, int64_t n, float *, hipStream_t)
{
    g_rec.M = n;
    return note(kLaunchAbsmax);
}

hipError_t launch_nvfp4(unsigned axis, bool two_d, const Nv4Args &a, hipStream_t)
{
    g_rec.axis = axis, g_rec.two_d = two_d, g_rec.nv = a;
    return note(kLaunchNv);
}

hipError_t launch_nvfp4_any(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                            hipStream_t)
{
    g_rec.axis = axis, g_rec.two_d = two_d, g_rec.nv = a, g_rec.gt = gt;
    return note(kLaunchNvAny);
}

hipError_t launch_nvfp4_grouped(unsigned axis, bool two_d, const Nv4Args &a,
                                const GroupTable &gt, hipStream_t)
{
    g_rec.axis = axis, g_rec.two_d = two_d, g_rec.nv = a, g_rec.gt = gt;
    return note(kLaunchNvGrouped);
}

hipError_t launch_nvfp4_ragged(unsigned axis, bool two_d, const Nv4Args &a,
                                const GroupTable &gt, hipStream_t)
{
    g_rec.axis = axis, g_rec.two_d = two_d, g_rec.nv = a, g_rec.gt = gt;
    return note(kLaunchNvRagged);
}

hipError_t launch_absmax_grouped(const uint16_t *, int64_t K, const GroupTable &gt, float *,
                                 hipStream_t)
{
    g_rec.K = K, g_rec.gt = gt;
    return note(kLaunchAbsmaxGrouped);
}

}  // namespace mxk
