// lowrank_fwd_bf16_vl.hip -- instantiates the low-rank fwd launchers for bf16
// on rows packed with documents (per-token positions).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, false, true>(const LrArgs &a);
}  // namespace dsc
