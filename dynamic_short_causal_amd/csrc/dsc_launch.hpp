// dsc_launch.hpp -- host-side interface between the C ABI (argument checks)
// and the kernel launchers.  Everything here has already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsc {

struct HwArgs {
  const void *x, *w, *dy;
  void *y, *dx, *dw;
  int64_t B, T, D;
  int W, H;
  bool bf16, residual, act, bwd;
  void *stream;
};

struct LrArgs {
  const void *x, *z, *U, *dy;
  void *y, *dx, *dz, *dU, *ws;
  int64_t B, T, D;
  int W, H, R;
  bool bf16, residual, act, bwd;
  void *stream;
};

// Tiling of the low-rank backward and the workspace it implies.  Shared by
// the workspace query and the launcher so the two always agree.
struct LrBwdPlan {
  int V;            // channels per 16-byte vector
  int gpv;          // filter groups per vector (V / H)
  int units;        // vectors per quarter-wave (channel units per wave)
  int64_t cb;       // channels per workgroup
  int64_t ncb;      // channel blocks
  int tc;           // tokens per workgroup chunk (multiple of 16)
  int64_t nchunk;   // chunks per sequence
  int64_t rpad;     // R padded to one 16-row MFMA block
  size_t dz_part;   // bytes of dz partials: ncb * B*T * rpad * 4
  size_t dU_part;   // bytes of dU partials: B*nchunk * rpad * G*W * 4
  size_t bytes;     // total workspace
};

inline LrBwdPlan lr_bwd_plan(int64_t B, int64_t T, int64_t D, int W, int H, int R,
                             bool bf16) {
  LrBwdPlan p{};
  p.V = bf16 ? 8 : 4;
  p.gpv = p.V / H;
  const int numax = W <= 3 ? 4 : W <= 6 ? 2 : 1;  // must match LrGeo::NU
  p.units = H < numax ? H : numax;   // channel vectors per lane
  p.cb = (int64_t)4 /*waves*/ * 4 /*quarters*/ * p.units * p.V;
  p.ncb = (D + p.cb - 1) / p.cb;
  p.rpad = 16;  // R <= 16: one 16-row MFMA block of ranks
  // Long chunks keep the dU partials small; enough workgroups to fill the
  // chip (>= 2 per CU) bound the length from above.
  int tc = 1024;
  while (tc > 16 && B * ((T + tc - 1) / tc) * p.ncb < 512) tc /= 2;
  if (T < tc) tc = (int)((T + 15) / 16 * 16);
  if (tc < 16) tc = 16;
  p.tc = tc;
  p.nchunk = (T + tc - 1) / tc;
  const int64_t G = D / H;
  p.dz_part = (size_t)p.ncb * (size_t)(B * T) * (size_t)p.rpad * 4;
  p.dU_part = (size_t)(B * p.nchunk) * (size_t)p.rpad * (size_t)(G * W) * 4;
  p.bytes = p.dz_part + p.dU_part;
  return p;
}

hipError_t headwise_launch(const HwArgs &a);
hipError_t lowrank_launch(const LrArgs &a);

}  // namespace dsc
