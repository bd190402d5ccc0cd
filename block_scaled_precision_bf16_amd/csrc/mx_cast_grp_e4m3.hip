// mx_cast_grp_e4m3.hip -- the grouped MXFP8 cast kernel instantiated for
// E4M3 elements, floor scale rule.
#include "mx_cast.h"

namespace mxk {
template hipError_t launch_mx_cast_fmt<0, true, false>(int, unsigned, bool, const MxArgs &,
                                                   const GroupTable *, hipStream_t);
}  // namespace mxk
