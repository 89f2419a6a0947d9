// lowrank_fwd_f32.hip -- instantiates the low-rank fwd launchers for float (plain rows) with
// DSC_LR_RB blocks of 16 ranks; build.py compiles it once per block count.
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch_rb<float, DSC_LR_RB, false, false>(const LrArgs &a);
}  // namespace dsc
