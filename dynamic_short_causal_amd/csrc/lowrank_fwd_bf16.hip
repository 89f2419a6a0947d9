// lowrank_fwd_bf16.hip -- instantiates the low-rank fwd launchers for bf16 (plain rows).
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, false, false>(const LrArgs &a);
}  // namespace dsc
