// lowrank_fwd_f32_vl.hip -- instantiates the low-rank fwd launchers for f32
// on rows packed with documents (per-token positions).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<float, false, true>(const LrArgs &a);
}  // namespace dsc
