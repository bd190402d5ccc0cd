// mx_cast_grp_e5m2.hip -- the grouped MXFP8 cast kernel instantiated for
// E5M2 elements, floor scale rule.
#include "mx_cast.h"

namespace mxk {
template hipError_t launch_mx_cast_fmt<kFmtE5M2, true, false>(int, unsigned, bool, const MxArgs &,
                                                   const GroupTable *, hipStream_t);
}  // namespace mxk
