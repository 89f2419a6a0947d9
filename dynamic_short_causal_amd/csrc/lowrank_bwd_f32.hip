// lowrank_bwd_f32.hip -- instantiates the low-rank bwd launchers for f32 (plain rows).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<float, true, false>(const LrArgs &a);
}  // namespace dsc
