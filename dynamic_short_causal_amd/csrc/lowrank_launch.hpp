// ---------------------------------------------------------------------------
// Host-side launchers, instantiated per dtype and direction in
// lowrank_{fwd,bwd}_{bf16,f32}.hip so the four parts compile in parallel.
// ---------------------------------------------------------------------------
#pragma once
#include <type_traits>
#include "lowrank_impl.hpp"
#include "lowrank_bwd_cl.hpp"
#include "lowrank_fwd_cl.hpp"
#include "lowrank_fwd_valu.hpp"

namespace dsc {

// the matrix-core forward (lr_fwd_kernel)
template <typename E, int W, int GPV, bool ACT, bool VL, int RB>
static hipError_t launch_lr_fwd_mfma(const LrArgs &a) {
  using Gm = LrGeo<E, W, GPV>;
  hipStream_t s = (hipStream_t)a.stream;
  const float rho = a.residual ? 1.f : 0.f;
  const int ncb = (int)((a.D + Gm::CB - 1) / Gm::CB);
  const int TC = pick_chunk(a.B, a.T, ncb, 768);  // 3 resident workgroups per CU
  const int nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t nblocks = a.B * nchunk * (int64_t)ncb;
  if (nblocks == 0) return hipSuccess;
  constexpr int smem = LrFwdGeo<E, W, GPV>::bytes;
  hipLaunchKernelGGL((lr_fwd_kernel<E, W, GPV, ACT, VL, RB>), dim3((unsigned)nblocks),
                     dim3(kLrThreads), smem, s, (const E *)a.x, (const E *)a.z,
                     (const E *)a.U, a.pos, (E *)a.y, (int)a.T, (int)a.D, a.R, TC, nchunk, ncb,
                     rho, lr_tie_multiple(a));
  return hipGetLastError();
}

// per-channel bf16 filters on plain rows, at most 16 ranks: one channel per
// lane (lowrank_fwd_cl.hpp), loads two 16-token steps ahead
constexpr int kLrFwdClPrefetch = 2;
template <int W, bool ACT>
static hipError_t launch_lr_fwd_cl(const LrArgs &a) {
  const int ncb = (int)((a.D + kClCB - 1) / kClCB);
  const int TC = pick_chunk(a.B, a.T, ncb, (int64_t)kLrClResident * 256);
  const int nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t nblocks = a.B * nchunk * (int64_t)ncb;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL((lr_fwd_cl_kernel<W, ACT, kLrFwdClPrefetch>), dim3((unsigned)nblocks),
                     dim3(kClThreads), LrFwdClGeo<W>::bytes, (hipStream_t)a.stream,
                     (const bf16 *)a.x, (const bf16 *)a.z, (const bf16 *)a.U, (bf16 *)a.y,
                     (int)a.T, (int)a.D, a.R, TC, nchunk, ncb, a.residual ? 1.f : 0.f);
  return hipGetLastError();
}

template <typename E, int W, int GPV, bool ACT, bool VL, int RB>
static hipError_t launch_lr_fwd(const LrArgs &a) {
  if constexpr (std::is_same_v<E, bf16> && GPV == 8 && RB == 1 && !VL) {
    if (a.H == 1 && a.R <= 16) return launch_lr_fwd_cl<W, ACT>(a);
  }
  // bf16 filters tied over 8 channels (one group per vector): vector ALUs
  if constexpr (std::is_same_v<E, bf16> && GPV == 1 && RB == 1 && W <= 4) {
    if (lr_fwd_uses_valu(a.bf16, a.D, a.W, a.H, a.R)) return launch_lr_fwd_valu<W, ACT, VL>(a);
  }
  return launch_lr_fwd_mfma<E, W, GPV, ACT, VL, RB>(a);
}

template <typename E>
static hipError_t launch_lr_reduce(const LrArgs &a, const LrBwdPlan &p, const float *dzp,
                                   const float *dUp);

// per-channel filters in bf16 without activation: one channel per lane
// (lowrank_bwd_cl.hpp)
template <int W, bool VL>
static hipError_t launch_lr_bwd_cl(const LrArgs &a) {
  hipStream_t s = (hipStream_t)a.stream;
  const float rho = a.residual ? 1.f : 0.f;
  const LrBwdPlan p = lr_bwd_plan(a.B, a.T, a.D, a.W, a.H, a.R, a.bf16, true);
  if (p.cb != kClCB || !lr_bwd_uses_cl(a.H, a.R, a.bf16, a.act)) return hipErrorInvalidValue;
  float *dzp = (float *)a.ws;
  float *dUp = (float *)((char *)a.ws + p.dz_part);
  const int64_t nblocks = a.B * p.nchunk * p.ncb;
  if (nblocks > 0) {
    constexpr int smem = LrBwdClGeo<W>::bytes;
    const int64_t N = a.B * a.T;
    hipLaunchKernelGGL((lr_bwd_cl_kernel<W, VL>), dim3((unsigned)nblocks), dim3(kClThreads),
                       smem, s, (const bf16 *)a.x, (const bf16 *)a.z, (const bf16 *)a.U,
                       (const bf16 *)a.dy, a.pos, (bf16 *)a.dx, dzp, dUp, (int)a.T, (int)a.D,
                       a.R, (int)p.tc, (int)p.nchunk, (int)p.ncb, N, rho);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_lr_reduce<bf16>(a, p, dzp, dUp);
}

// One launch of lr_bwd_kernel per block of 16 ranks (the first also writes
// dx), then the fixed-order reduction of every block's partials.
template <typename E, int W, int GPV, bool VL, int RB>
static hipError_t launch_lr_bwd(const LrArgs &a) {
  if (RB == 1 && lr_bwd_uses_cl(a.H, a.R, sizeof(E) == 2, a.act)) {  // bf16, H = 1, R <= 16, no SiLU
    return launch_lr_bwd_cl<W, VL>(a);
  } else {
    hipStream_t s = (hipStream_t)a.stream;
    const float rho = a.residual ? 1.f : 0.f;
    const LrBwdPlan p = lr_bwd_plan(a.B, a.T, a.D, a.W, a.H, a.R, a.bf16, false);
    const int64_t N = a.B * a.T;
    float *dzp = (float *)a.ws;
    float *dUp = (float *)((char *)a.ws + p.dz_part);
    const int64_t nblocks = a.B * p.nchunk * p.ncb;
    for (int rb0 = 0; nblocks > 0 && rb0 < RB; ++rb0) {
      constexpr int smem = LrBwdGeo<E, W, GPV, RB>::bytes;
      hipLaunchKernelGGL((lr_bwd_kernel<E, W, GPV, VL, RB>), dim3((unsigned)nblocks),
                         dim3(kLrThreads), smem, s, (const E *)a.x, (const E *)a.z,
                         (const E *)a.U, (const E *)a.dy, a.pos, (E *)a.dx, dzp, dUp,
                         (int)a.T, (int)a.D, a.R, p.tc, (int)p.nchunk, (int)p.ncb, N, rho,
                         a.act ? 1 : 0, rb0, rb0 == 0 ? 1 : 0, lr_tie_multiple(a));
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return launch_lr_reduce<E>(a, p, dzp, dUp);
  }
}

// fixed-order sums of the dz and dU partials, cast to the output type
template <typename E>
static hipError_t launch_lr_reduce(const LrArgs &a, const LrBwdPlan &p, const float *dzp,
                                   const float *dUp) {
  hipStream_t s = (hipStream_t)a.stream;
  const int64_t N = a.B * a.T;
  const int64_t GW = (a.D / a.H) * a.W;
  const int hm = lr_tie_multiple(a);
  // four outputs per thread where R and G*W allow it (16-byte partial loads)
  const bool by4 = a.R % 4 == 0 && GW % 4 == 0 && hm == 1;
  const int64_t total = (N * a.R + (int64_t)a.R * GW) / (by4 ? 4 : 1);
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  if (by4)
    hipLaunchKernelGGL((lr_reduce4_kernel<E>), dim3((unsigned)grid), dim3(256), 0, s, dzp, dUp,
                       (E *)a.dz, (E *)a.dU, N, a.R, (int)p.rpad, (int)p.ncb, GW,
                       (int)(a.B * p.nchunk));
  else
    hipLaunchKernelGGL((lr_reduce_kernel<E>), dim3((unsigned)grid), dim3(256), 0, s, dzp, dUp,
                       (E *)a.dz, (E *)a.dU, N, a.R, (int)p.rpad, (int)p.ncb, GW,
                       (int)(a.B * p.nchunk), a.W, hm);
  return hipGetLastError();
}

// RB blocks of 16 ranks (the dispatcher picks RB = 1, 2 or 4 for R <= 16, 32, 64)
template <typename E, int W, int GPV, int RB, bool BWD, bool VL>
static hipError_t lr_rb(const LrArgs &a) {
  if constexpr (BWD) {
    return launch_lr_bwd<E, W, GPV, VL, RB>(a);
  } else {
    return a.act ? launch_lr_fwd<E, W, GPV, true, VL, RB>(a)
                 : launch_lr_fwd<E, W, GPV, false, VL, RB>(a);
  }
}

template <typename E, int W, int RB, bool BWD, bool VL>
static hipError_t lr_gpv(const LrArgs &a) {
  constexpr int V = Vw<E>::n;
  // groups per vector; filters tied over several vectors tile as one group
  // per vector (lr_tie_multiple)
  switch (a.H >= V ? 1 : V / a.H) {
    case 1: return lr_rb<E, W, 1, RB, BWD, VL>(a);
    case 2: return lr_rb<E, W, 2, RB, BWD, VL>(a);
    case 4: return lr_rb<E, W, 4, RB, BWD, VL>(a);
    default:
      if constexpr (V == 8) return lr_rb<E, W, 8, RB, BWD, VL>(a);
      return hipErrorInvalidValue;
  }
}

// VL: rows packed with documents (a.pos set).  Each (dtype, direction, VL,
// RB) set is instantiated in a translation unit of its own so they compile
// in parallel.
template <typename E, int RB, bool BWD, bool VL>
hipError_t lr_dispatch_rb(const LrArgs &a) {
  switch (a.W) {
    case 1: return lr_gpv<E, 1, RB, BWD, VL>(a);
    case 2: return lr_gpv<E, 2, RB, BWD, VL>(a);
    case 3: return lr_gpv<E, 3, RB, BWD, VL>(a);
    case 4: return lr_gpv<E, 4, RB, BWD, VL>(a);
    case 5: return lr_gpv<E, 5, RB, BWD, VL>(a);
    case 6: return lr_gpv<E, 6, RB, BWD, VL>(a);
    case 7: return lr_gpv<E, 7, RB, BWD, VL>(a);
    case 8: return lr_gpv<E, 8, RB, BWD, VL>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsc
