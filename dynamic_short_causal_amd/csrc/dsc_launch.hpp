// dsc_launch.hpp -- host-side interface between the C ABI (argument checks)
// and the kernel launchers.  Everything here has already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsc {

// pos: optional int32 (B, T) document positions of packed rows (tap k of
// token t is used only when k <= pos[b,t]); nullptr for plain rows.
struct HwArgs {
  const void *x, *w, *dy;
  const int32_t *pos;
  void *y, *dx, *dw;
  int64_t B, T, D;
  int W, H;
  bool bf16, residual, act, bwd;
  void *stream;
};

struct LrArgs {
  const void *x, *z, *U, *dy;
  const int32_t *pos;  // as in HwArgs
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

// Token-chunk length of a (batch, chunk, channel block) grid.  Long chunks
// amortise per-workgroup set-up and keep the partial sums few; the grid should
// also fill whole rounds of `resident` concurrent workgroups (MI355X: 256
// CUs), since a last, partial round leaves CUs idle.  Picks the longest power
// of two in 64..2048 whose rounds are at least 90 % full, else the fullest.
inline int pick_chunk(int64_t B, int64_t T, int64_t ncb, int64_t resident) {
  int best = 64;
  double best_eff = -1.0;
  for (int tc = 2048; tc >= 64; tc /= 2) {
    const int64_t wg = B * ((T + tc - 1) / tc) * ncb;
    if (wg <= 0) return (int)((T + 15) / 16 * 16);
    const int64_t rounds = (wg + resident - 1) / resident;
    const double eff = (double)wg / (double)(rounds * resident);
    if (eff >= 0.9) { best = tc; break; }
    if (eff > best_eff + 1e-9) { best_eff = eff; best = tc; }
  }
  if (T < best) best = (int)((T + 15) / 16 * 16);
  return best < 16 ? 16 : best;
}

inline LrBwdPlan lr_bwd_plan(int64_t B, int64_t T, int64_t D, int W, int H, int R,
                             bool bf16) {
  LrBwdPlan p{};
  p.V = bf16 ? 8 : 4;
  p.gpv = p.V / H;
  p.units = 1;  // channel vectors per lane (LrGeo::NU)
  p.cb = (int64_t)4 /*waves*/ * 4 /*quarters*/ * p.units * p.V;
  p.ncb = (D + p.cb - 1) / p.cb;
  p.rpad = 16;  // R <= 16: one 16-row MFMA block of ranks
  p.tc = pick_chunk(B, T, p.ncb, 768);  // 3 resident workgroups per CU
  p.nchunk = (T + p.tc - 1) / p.tc;
  const int64_t G = D / H;
  p.dz_part = (size_t)p.ncb * (size_t)(B * T) * (size_t)p.rpad * 4;
  p.dU_part = (size_t)(B * p.nchunk) * (size_t)p.rpad * (size_t)(G * W) * 4;
  p.bytes = p.dz_part + p.dU_part;
  return p;
}

hipError_t headwise_launch(const HwArgs &a);
hipError_t lowrank_launch(const LrArgs &a);

}  // namespace dsc
