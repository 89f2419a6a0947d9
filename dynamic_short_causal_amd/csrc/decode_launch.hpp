// decode_launch.hpp -- host-side arguments of the one-token (decode) kernels
// in decode.hip, filled in by the C ABI after its checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsc {

// Head-wise uses w (B, G, W); low-rank uses z (B, R) and U (R, G*W); the
// state is (B, W-1, D).  decode_state_launch reads x as a prompt (B, T, D).
struct DecArgs {
  const void *x, *w, *z, *U;
  void *state, *y;
  int64_t B, T, D;
  int W, H, R;
  bool bf16, residual, act, lowrank;
  void *stream;
};

hipError_t decode_launch(const DecArgs &a);
hipError_t decode_state_launch(const DecArgs &a);

}  // namespace dsc
