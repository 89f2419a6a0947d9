// lowrank.hip -- entry of the low-rank launchers (see lowrank_impl.hpp for the
// kernels and lowrank_launch.hpp for the tiling and dispatch): picks the
// instance set for the dtype, direction, packed rows and rank blocks.
#include "dsc_device.hpp"
#include "dsc_launch.hpp"

namespace dsc {

template <typename E, int RB, bool BWD, bool VL> hipError_t lr_dispatch_rb(const LrArgs &a);
#define DSC_LR_EXTERN(E, RB)                                                   \
  extern template hipError_t lr_dispatch_rb<E, RB, false, false>(const LrArgs &a); \
  extern template hipError_t lr_dispatch_rb<E, RB, true, false>(const LrArgs &a);  \
  extern template hipError_t lr_dispatch_rb<E, RB, false, true>(const LrArgs &a);  \
  extern template hipError_t lr_dispatch_rb<E, RB, true, true>(const LrArgs &a);
DSC_LR_EXTERN(bf16, 1)
DSC_LR_EXTERN(bf16, 2)
DSC_LR_EXTERN(bf16, 4)
DSC_LR_EXTERN(float, 1)
DSC_LR_EXTERN(float, 2)
DSC_LR_EXTERN(float, 4)
#undef DSC_LR_EXTERN

template <typename E, bool BWD, bool VL>
static hipError_t lr_dispatch(const LrArgs &a) {
  switch (lr_rank_blocks(a.R)) {
    case 1: return lr_dispatch_rb<E, 1, BWD, VL>(a);
    case 2: return lr_dispatch_rb<E, 2, BWD, VL>(a);
    default: return lr_dispatch_rb<E, 4, BWD, VL>(a);
  }
}

template <bool VL>
static hipError_t lowrank_vl(const LrArgs &a) {
  if (a.bf16) return a.bwd ? lr_dispatch<bf16, true, VL>(a) : lr_dispatch<bf16, false, VL>(a);
  return a.bwd ? lr_dispatch<float, true, VL>(a) : lr_dispatch<float, false, VL>(a);
}

hipError_t lowrank_launch(const LrArgs &a) {
  if (!a.bwd && (a.B == 0 || a.T == 0)) return hipSuccess;
  return a.pos ? lowrank_vl<true>(a) : lowrank_vl<false>(a);
}

}  // namespace dsc
