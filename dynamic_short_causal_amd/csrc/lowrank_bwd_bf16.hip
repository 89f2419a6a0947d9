// lowrank_bwd_bf16.hip -- instantiates the low-rank bwd launchers for bf16 (plain rows).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, true, false>(const LrArgs &a);
}  // namespace dsc
