// lowrank_bwd_bf16.hip -- instantiates the low-rank bwd launchers for bf16 (plain rows) with
// DSC_LR_RB blocks of 16 ranks; build.py compiles it once per block count.
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch_rb<bf16, DSC_LR_RB, true, false>(const LrArgs &a);
}  // namespace dsc
