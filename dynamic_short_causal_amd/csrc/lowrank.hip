// lowrank.hip -- placeholder until the low-rank kernels land.
#include "dsc_launch.hpp"
namespace dsc {
hipError_t lowrank_launch(const LrArgs &) { return hipErrorNotSupported; }
}  // namespace dsc
