// lowrank_fwd_f32.hip -- instantiates the low-rank fwd launchers for f32.
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<float, false>(const LrArgs &a);
}  // namespace dsc
