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

// Filters tied over hm whole channel vectors (H = hm * vector width): the
// low-rank kernels then tile one group per vector and read U's column of
// group c / H.  1 when a vector holds one or more groups.
inline int lr_tie_multiple(const LrArgs &a) {
  const int V = a.bf16 ? 8 : 4;
  return a.H > V ? a.H / V : 1;
}

// Workgroup shape of the low-rank backward for per-channel bf16 filters without
// activation (lr_bwd_cl_kernel): waves, 16-channel groups per wave, and the
// workgroups resident on one CU.
constexpr int kLrClWaves = 4;
constexpr int kLrClNG = 2;
constexpr int kLrClCB = 16 * kLrClNG * kLrClWaves;
constexpr int kLrClResident = 3;

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
  int64_t rpad;     // R padded to whole 16-row MFMA blocks
  size_t dz_part;   // bytes of dz partials: ncb * B*T * rpad * 4
  size_t dU_part;   // bytes of dU partials: B*nchunk * rpad * G*W * 4
  size_t bytes;     // total workspace
};

// Token-chunk length of a (batch, chunk, channel block) grid.  Long chunks
// amortise per-workgroup set-up and keep the partial sums few; the grid should
// also fill whole rounds of `resident` concurrent workgroups (MI355X: 256
// CUs), since a last, partial round leaves CUs idle.  Picks the longest power
// of two in 64..2048 whose rounds are at least 90 % full, else the fullest.
// Never below 16 (one tile), also for an empty grid, so that the chunk count
// (T + tc - 1) / tc is always defined.
inline int pick_chunk(int64_t B, int64_t T, int64_t ncb, int64_t resident) {
  if (B <= 0 || T <= 0 || ncb <= 0) return 16;
  int best = 64;
  double best_eff = -1.0;
  for (int tc = 2048; tc >= 64; tc /= 2) {
    const int64_t wg = B * ((T + tc - 1) / tc) * ncb;
    const int64_t rounds = (wg + resident - 1) / resident;
    const double eff = (double)wg / (double)(rounds * resident);
    if (eff >= 0.9) { best = tc; break; }
    if (eff > best_eff + 1e-9) { best_eff = eff; best = tc; }
  }
  if (T < best) best = (int)((T + 15) / 16 * 16);
  return best < 16 ? 16 : best;
}

// Blocks of 16 ranks the low-rank kernels are built for: 1, 2 or 4.
inline int lr_rank_blocks(int R) { return R <= 16 ? 1 : R <= 32 ? 2 : 4; }

// The kernel a low-rank backward call runs: per-channel bf16 filters of at
// most 16 ranks without activation take lr_bwd_cl_kernel, everything else
// lr_bwd_kernel.
inline bool lr_bwd_uses_cl(int H, int R, bool bf16, bool act) {
  return bf16 && H == 1 && R <= 16 && !act;
}

inline LrBwdPlan lr_bwd_plan(int64_t B, int64_t T, int64_t D, int W, int H, int R, bool bf16,
                             bool cl) {
  LrBwdPlan p{};
  p.V = bf16 ? 8 : 4;
  p.gpv = H >= p.V ? 1 : p.V / H;
  p.units = 1;  // channel vectors per lane (LrGeo::NU)
  p.cb = cl ? kLrClCB : (int64_t)4 /*waves*/ * 4 /*quarters*/ * p.units * p.V;
  p.ncb = (D + p.cb - 1) / p.cb;
  p.rpad = 16 * lr_rank_blocks(R);  // whole 16-row MFMA blocks of ranks
  p.tc = pick_chunk(B, T, p.ncb, (cl ? kLrClResident : 3) * 256);
  p.nchunk = (T + p.tc - 1) / p.tc;
  // groups of a dU partial row: those of the kernels' tiling, one per vector
  // when the filters are tied over several vectors
  const int64_t G = D / (H > p.V ? p.V : H);
  p.dz_part = (size_t)p.ncb * (size_t)(B * T) * (size_t)p.rpad * 4;
  p.dU_part = (size_t)(B * p.nchunk) * (size_t)p.rpad * (size_t)(G * W) * 4;
  p.bytes = p.dz_part + p.dU_part;
  return p;
}

// Workspace of a low-rank backward call with or without activation (the
// query takes no flags): the larger need of the kernels the shape can take.
inline size_t lr_bwd_workspace(int64_t B, int64_t T, int64_t D, int W, int H, int R, bool bf16) {
  const size_t g = lr_bwd_plan(B, T, D, W, H, R, bf16, false).bytes;
  if (!lr_bwd_uses_cl(H, R, bf16, false)) return g;
  const size_t c = lr_bwd_plan(B, T, D, W, H, R, bf16, true).bytes;
  return c > g ? c : g;
}

hipError_t headwise_launch(const HwArgs &a);
hipError_t lowrank_launch(const LrArgs &a);

}  // namespace dsc
