// gen_launch.hpp -- host-side arguments of the fused filter-generation kernel
// in gen.hip (head-wise forward with w = xh M formed on chip), filled in by
// the C ABI after its checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsc {

// x, y (B, T, D); xh (B, T, Dh); Mt (G*W, Dh): row g*W + k holds column
// g*W + k of M; bf16 only.
struct GenArgs {
  const void *x, *xh, *Mt;
  void *y;
  int64_t B, T, D, Dh;
  int W, H;
  bool residual, act;
  void *stream;
};

hipError_t gen_launch(const GenArgs &a);

}  // namespace dsc
