// lowrank.hip -- entry of the low-rank launchers (see lowrank_impl.hpp for the
// kernels and lowrank_launch.hpp for the tiling and dispatch).
#include "dsc_device.hpp"
#include "dsc_launch.hpp"

namespace dsc {

template <typename E, bool BWD, bool VL> hipError_t lr_dispatch(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, false, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, true, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, false, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, true, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, false, true>(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, true, true>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, false, true>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, true, true>(const LrArgs &a);

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
