// mx_cast_rag_e4m3_up.hip -- the grouped MXFP8 cast kernel for transposed rows
// that start at any byte, instantiated for E4M3 elements, round-up scale rule.
#include "mx_cast.h"

namespace mxk {
template hipError_t launch_mx_cast_fmt<kFmtRoundUp, true, true>(int, unsigned, bool, const MxArgs &,
                                                   const GroupTable *, hipStream_t);
}  // namespace mxk
