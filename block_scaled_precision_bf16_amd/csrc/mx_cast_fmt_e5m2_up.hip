// mx_cast_fmt_e5m2_up.hip -- the MXFP8 cast kernel instantiated for E5M2 elements, round-up scale rule.
#include "mx_cast.h"

namespace mxk {
template hipError_t launch_mx_cast_fmt<kFmtE5M2 | kFmtRoundUp, false, false>(int, unsigned, bool, const MxArgs &,
                                                    const GroupTable *, hipStream_t);
}  // namespace mxk
