// lowrank_fwd_bf16.hip -- instantiates the low-rank fwd launchers for bf16.
#include "lowrank_launch.hpp"

namespace dsc {
template hipError_t lr_dispatch<bf16, false>(const LrArgs &a);
}  // namespace dsc
