// lowrank_bwd_bf16_vl.hip -- instantiates the low-rank bwd launchers for bf16
// on rows packed with documents (per-token positions).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, true, true>(const LrArgs &a);
}  // namespace dsc
