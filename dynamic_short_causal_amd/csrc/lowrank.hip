// lowrank.hip -- entry of the low-rank launchers (see lowrank_impl.hpp for the
// kernels and lowrank_launch.hpp for the tiling and dispatch).
#include "dsc_device.hpp"
#include "dsc_launch.hpp"

namespace dsc {

template <typename E, bool BWD> hipError_t lr_dispatch(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<bf16, true>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, false>(const LrArgs &a);
extern template hipError_t lr_dispatch<float, true>(const LrArgs &a);

hipError_t lowrank_launch(const LrArgs &a) {
  if (!a.bwd && (a.B == 0 || a.T == 0)) return hipSuccess;
  if (a.bf16) return a.bwd ? lr_dispatch<bf16, true>(a) : lr_dispatch<bf16, false>(a);
  return a.bwd ? lr_dispatch<float, true>(a) : lr_dispatch<float, false>(a);
}

}  // namespace dsc
