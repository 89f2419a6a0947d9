// lowrank_bwd_bf16.hip -- instantiates the low-rank bwd launchers for bf16.
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, true>(const LrArgs &a);
}  // namespace dsc
