// ---------------------------------------------------------------------------
// Host-side launchers, instantiated per dtype and direction in
// lowrank_{fwd,bwd}_{bf16,f32}.hip so the four parts compile in parallel.
// ---------------------------------------------------------------------------
#pragma once
#include "lowrank_impl.hpp"
#include "lowrank_bwd_cl.hpp"

namespace dsc {

template <typename E, int W, int GPV, bool ACT, bool VL>
static hipError_t launch_lr_fwd(const LrArgs &a) {
  using Gm = LrGeo<E, W, GPV>;
  hipStream_t s = (hipStream_t)a.stream;
  const float rho = a.residual ? 1.f : 0.f;
  const int ncb = (int)((a.D + Gm::CB - 1) / Gm::CB);
  const int TC = pick_chunk(a.B, a.T, ncb, 768);  // 3 resident workgroups per CU
  const int nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t nblocks = a.B * nchunk * (int64_t)ncb;
  if (nblocks == 0) return hipSuccess;
  constexpr int smem = LrFwdGeo<E, W, GPV>::bytes;
  hipLaunchKernelGGL((lr_fwd_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                     dim3(kLrThreads), smem, s, (const E *)a.x, (const E *)a.z,
                     (const E *)a.U, a.pos, (E *)a.y, (int)a.T, (int)a.D, a.R, TC, nchunk, ncb,
                     rho);
  return hipGetLastError();
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
  const LrBwdPlan p = lr_bwd_plan(a.B, a.T, a.D, a.W, a.H, a.R, a.bf16);
  if (p.cb != kClCB || a.H != 1 || a.act) return hipErrorInvalidValue;
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

template <typename E, int W, int GPV, bool VL>
static hipError_t launch_lr_bwd(const LrArgs &a) {
  if (sizeof(E) == 2 && GPV == 8 && !a.act) {  // H == 1, no SiLU
    return launch_lr_bwd_cl<W, VL>(a);
  } else {
    hipStream_t s = (hipStream_t)a.stream;
    const float rho = a.residual ? 1.f : 0.f;
    const LrBwdPlan p = lr_bwd_plan(a.B, a.T, a.D, a.W, a.H, a.R, a.bf16);
    const int64_t N = a.B * a.T;
    float *dzp = (float *)a.ws;
    float *dUp = (float *)((char *)a.ws + p.dz_part);
    const int64_t nblocks = a.B * p.nchunk * p.ncb;
    if (nblocks > 0) {
      constexpr int smem = LrBwdGeo<E, W, GPV>::bytes;
      hipLaunchKernelGGL((lr_bwd_kernel<E, W, GPV, VL>), dim3((unsigned)nblocks),
                         dim3(kLrThreads), smem, s, (const E *)a.x, (const E *)a.z,
                         (const E *)a.U, (const E *)a.dy, a.pos, (E *)a.dx, dzp, dUp,
                         (int)a.T, (int)a.D, a.R, p.tc, (int)p.nchunk, (int)p.ncb, N, rho,
                         a.act ? 1 : 0);
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
  const int64_t total = N * a.R + (int64_t)a.R * GW;
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((lr_reduce_kernel<E>), dim3((unsigned)grid), dim3(256), 0, s, dzp, dUp,
                     (E *)a.dz, (E *)a.dU, N, a.R, (int)p.rpad, (int)p.ncb, GW,
                     (int)(a.B * p.nchunk));
  return hipGetLastError();
}

// one 16-row rank block: the argument checks admit R <= 16 only
template <typename E, int W, int GPV, bool BWD, bool VL>
static hipError_t lr_rb(const LrArgs &a) {
  if constexpr (BWD) {
    return launch_lr_bwd<E, W, GPV, VL>(a);
  } else {
    return a.act ? launch_lr_fwd<E, W, GPV, true, VL>(a) : launch_lr_fwd<E, W, GPV, false, VL>(a);
  }
}

template <typename E, int W, bool BWD, bool VL>
static hipError_t lr_gpv(const LrArgs &a) {
  constexpr int V = Vw<E>::n;
  switch (V / a.H) {
    case 1: return lr_rb<E, W, 1, BWD, VL>(a);
    case 2: return lr_rb<E, W, 2, BWD, VL>(a);
    case 4: return lr_rb<E, W, 4, BWD, VL>(a);
    default:
      if constexpr (V == 8) return lr_rb<E, W, 8, BWD, VL>(a);
      return hipErrorInvalidValue;
  }
}

// VL: rows packed with documents (a.pos set); instantiated in their own
// translation units so the two builds compile in parallel
template <typename E, bool BWD, bool VL>
hipError_t lr_dispatch(const LrArgs &a) {
  switch (a.W) {
    case 1: return lr_gpv<E, 1, BWD, VL>(a);
    case 2: return lr_gpv<E, 2, BWD, VL>(a);
    case 3: return lr_gpv<E, 3, BWD, VL>(a);
    case 4: return lr_gpv<E, 4, BWD, VL>(a);
    case 5: return lr_gpv<E, 5, BWD, VL>(a);
    case 6: return lr_gpv<E, 6, BWD, VL>(a);
    case 7: return lr_gpv<E, 7, BWD, VL>(a);
    case 8: return lr_gpv<E, 8, BWD, VL>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsc
