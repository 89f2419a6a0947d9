// lowrank_fwd_f32.hip -- instantiates the low-rank fwd launchers for f32 (plain rows).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<float, false, false>(const LrArgs &a);
}  // namespace dsc
