// headwise.hip -- gfx950 kernels of the head-wise dynamic short convolution.
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (bullets
// Mechanisme, Parametrisatie 2 "head-wise tying", Plaatsing "residual").
// The backward is the derivative of that forward.
//
// Mapping (both kernels): one lane owns one 16-byte vector of channels (8 bf16
// or 4 fp32) and walks a chunk of TC consecutive tokens of one sequence.  A
// 64-lane wave therefore reads 1 KiB of one token row per instruction, fully
// coalesced; the W-1 previous rows of the causal window stay in registers, so
// each x row is fetched once per chunk plus a (W-1)-row halo at the chunk
// start.  Lanes of one filter group fetch the same filter row (merged by the
// cache); when a group spans L > 1 lanes the filter gradient is summed across
// those lanes with shuffles, and the backward gives each wave 64 / L whole
// groups (lanes past them idle when L is not a power of two).  Every output
// element has one writer.
//
// Packed rows (VL): with document positions pos (B, T), the taps of token t
// beyond pos[b,t] are zeroed before use, which removes every term that would
// reach into the previous document, in the forward, in dx and in dw alike.
// pos is uniform across a wave (one token at a time), so it is a scalar load.
//
// Cache policy: x, w, dy are read and y, dx written once per call, so they
// are all loaded and stored non-temporally (measured on MI355X with inputs
// that are not cache-resident: 3 % faster forward, 9 % faster backward).
#include "dsc_device.hpp"
#include "dsc_launch.hpp"

namespace dsc {

constexpr int kThreads = 256;

// Group geometry of one lane's vector.  GPV > 1: the vector holds GPV whole
// groups of H = V / GPV channels.  GPV == 1: the vector lies inside one group
// (H >= V); L = H / V lanes share it.
template <typename E, int GPV> struct Geo {
  static constexpr int V = Vw<E>::n;
  static constexpr int HS = V / GPV;  // channels per group inside the vector
};

// ---------------------------------------------------------------------------
// Forward: y[t] = act(sum_k w[t,g,k] x[t-k]) + rho x[t]
// ---------------------------------------------------------------------------
// zero the taps of a token beyond its document position p (packed rows); tap
// 0 always stays, so a negative p acts as 0
template <int W, int NG>
__device__ __forceinline__ void mask_taps(float (&taps)[NG * W], int p) {
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int k = 1; k < W; ++k)
      if (k > p) taps[gi * W + k] = 0.f;
}

template <typename E, int W, int GPV, bool ACT, bool VL>
__global__ __launch_bounds__(kThreads) void hw_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, const int32_t *__restrict__ pos,
    E *__restrict__ y, int T, int64_t D, int64_t G, int H, int nvec, int nvb, int TC,
    int nchunk, float rho) {
  constexpr int V = Vw<E>::n;
  constexpr int UN = 4;  // tokens loaded ahead per step
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int v = vb * kThreads + threadIdx.x;
  if (v >= nvec) return;

  const int t0 = chunk * TC;
  const int t1 = min(T, t0 + TC);
  const int64_t c0 = (int64_t)v * V;
  const int g0 = (v * V) / H;  // first group of this vector (D < 2^31)
  const E *xp = x + (int64_t)b * T * D + c0;
  E *yp = y + (int64_t)b * T * D + c0;
  const E *wp = w + ((int64_t)b * T * G + g0) * W;
  const int64_t wstride = G * W;

  // win[k] = x_{t-k} while token t is processed.  Each step first shifts the
  // window by one and then loads x_t into win[0], so before the first step
  // win[k-1] holds x_{t0-k} (zero before the sequence start).
  float win[W][V];
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int tt = t0 - k;
    if (tt >= 0) {
      unpack<E>(ld16nt(xp + (int64_t)tt * D), win[k - 1]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) win[k - 1][i] = 0.f;
    }
  }

  for (int t = t0; t < t1; t += UN) {
    uint4 xr[UN];
    RowBits<E, GPV * W> wr[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (t + u < t1) {
        xr[u] = ld16nt(xp + (int64_t)(t + u) * D);
        wr[u] = ld_row<E, GPV * W, true>(wp + (int64_t)(t + u) * wstride);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (t + u < t1) {
#pragma unroll
        for (int k = W - 1; k > 0; --k)
#pragma unroll
          for (int i = 0; i < V; ++i) win[k][i] = win[k - 1][i];
        unpack<E>(xr[u], win[0]);
        float taps[GPV * W];
        unpack_row<E, GPV * W>(wr[u], taps);
        if constexpr (VL) mask_taps<W, GPV>(taps, pos[(int64_t)b * T + t + u]);
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int gi = i / Geo<E, GPV>::HS;
          float s = 0.f;
#pragma unroll
          for (int k = 0; k < W; ++k) s = fmaf(taps[gi * W + k], win[k][i], s);
          if constexpr (ACT) s = silu_f(s);
          o[i] = fmaf(rho, win[0][i], s);
        }
        st16nt(yp + (int64_t)(t + u) * D, pack<E>(o));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward: ds = dy act'(s);  dx[tau] = sum_k w[tau+k,g,k] ds[tau+k] + rho dy[tau];
//           dw[t,g,k] = sum_{c in g} ds[t,c] x[t-k,c]
// The lane walks t = t0 .. t1+W-2.  acc[j] holds the partial dx of token
// t-1-j; token t adds w[t,g,k] ds[t] to token t-k, after which token t-W+1 is
// complete and is stored.  Tokens t1 .. t1+W-2 (the right halo) only feed dx.
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT, bool VL>
__device__ __forceinline__ void hw_bwd_token(
    const E *xp, const E *dyp, const E *wp, E *dxp, E *dwp, int64_t D,
    int64_t wstride, int t, int t0, int t1, int T, int L, int lane_in_group,
    float rho, float (&win)[W][Geo<E, GPV>::V], float (&acc)[W > 1 ? W - 1 : 1][Geo<E, GPV>::V],
    uint4 xr, uint4 dyr, const RowBits<E, GPV * W> &wr, int p) {
  constexpr int V = Vw<E>::n;
  constexpr int HS = Geo<E, GPV>::HS;
  const bool in_chunk = t < t1;
  const bool in_seq = t < T;
#pragma unroll
  for (int k = W - 1; k > 0; --k)
#pragma unroll
    for (int i = 0; i < V; ++i) win[k][i] = win[k - 1][i];
  float dyv[V], ds[V], taps[GPV * W];
  if (in_seq) {
    unpack<E>(dyr, dyv);
    unpack_row<E, GPV * W>(wr, taps);
    if constexpr (VL) mask_taps<W, GPV>(taps, p);
    if (ACT || in_chunk) {
      unpack<E>(xr, win[0]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) win[0][i] = 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) { dyv[i] = 0.f; win[0][i] = 0.f; }
#pragma unroll
    for (int j = 0; j < GPV * W; ++j) taps[j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if constexpr (ACT) {
      const int gi = i / HS;
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) s = fmaf(taps[gi * W + k], win[k][i], s);
      ds[i] = dyv[i] * silu_grad_f(s);
    } else {
      ds[i] = dyv[i];
    }
  }
  // filter gradient of token t (inside the chunk only)
  if (in_chunk) {
    float pw[GPV][W];
#pragma unroll
    for (int gi = 0; gi < GPV; ++gi)
#pragma unroll
      for (int k = 0; k < W; ++k) {
        float a = 0.f;
#pragma unroll
        for (int h = 0; h < HS; ++h) a = fmaf(ds[gi * HS + h], win[k][gi * HS + h], a);
        pw[gi][k] = (VL && k > 0 && k > p) ? 0.f : a;
      }
    if constexpr (GPV == 1) group_sum<W>(pw[0], L, lane_in_group);
    if (GPV > 1 || lane_in_group == 0) {
      float flat[GPV * W];
#pragma unroll
      for (int gi = 0; gi < GPV; ++gi)
#pragma unroll
        for (int k = 0; k < W; ++k) flat[gi * W + k] = pw[gi][k];
      st_row<E, GPV * W>(dwp + (int64_t)t * wstride, flat);
    }
  }
  // input gradient: token t contributes to tokens t, t-1, ..., t-W+1
  float o[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int gi = i / HS;
    const float cur = fmaf(taps[gi * W], ds[i], rho * dyv[i]);  // token t itself
    if constexpr (W == 1) {
      o[i] = cur;
    } else {
#pragma unroll
      for (int k = 1; k < W; ++k) acc[k - 1][i] = fmaf(taps[gi * W + k], ds[i], acc[k - 1][i]);
      o[i] = acc[W - 2][i];  // token t-W+1, now complete
#pragma unroll
      for (int j = W - 2; j > 0; --j) acc[j][i] = acc[j - 1][i];
      acc[0][i] = cur;
    }
  }
  const int tau = t - (W - 1);
  if (tau >= t0 && tau < t1) st16nt(dxp + (int64_t)tau * D, pack<E>(o));
}

template <typename E, int W, int GPV, bool ACT, bool VL>
__global__ __launch_bounds__(kThreads) void hw_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, const E *__restrict__ dy,
    const int32_t *__restrict__ pos, E *__restrict__ dx, E *__restrict__ dw, int T, int64_t D,
    int64_t G, int H, int nvec, int nvb, int TC, int nchunk, float rho, int U) {
  constexpr int V = Vw<E>::n;
  constexpr int UN = 4;
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  // Each wave takes U = 64 / L * L consecutive vectors, whole groups of L
  // lanes (U = 64 when L is a power of two); nvec is a multiple of L, so whole
  // groups retire together and the shuffles never mix active and idle lanes.
  const int lane = threadIdx.x & 63;
  if (lane >= U) return;
  const int v = (vb * (kThreads / 64) + (int)(threadIdx.x >> 6)) * U + lane;
  if (v >= nvec) return;

  const int t0 = chunk * TC;
  const int t1 = min(T, t0 + TC);
  const int64_t c0 = (int64_t)v * V;
  const int g0 = (v * V) / H;
  const int L = (GPV == 1) ? H / V : 1;
  const int lane_in_group = (GPV == 1) ? (lane % L) : 0;
  const int64_t base = (int64_t)b * T * D + c0;
  const E *xp = x + base;
  const E *dyp = dy + base;
  E *dxp = dx + base;
  const int64_t wbase = ((int64_t)b * T * G + g0) * W;
  const E *wp = w + wbase;
  E *dwp = dw + wbase;
  const int64_t wstride = G * W;

  float win[W][V];
  float acc[W > 1 ? W - 1 : 1][V];
#pragma unroll
  for (int j = 0; j < (W > 1 ? W - 1 : 1); ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[j][i] = 0.f;
  // window as in the forward: win[k-1] = x_{t0-k} before the first step
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int tt = t0 - k;
    if (tt >= 0) {
      unpack<E>(ld16nt(xp + (int64_t)tt * D), win[k - 1]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) win[k - 1][i] = 0.f;
    }
  }
  // main chunk
  for (int t = t0; t < t1; t += UN) {
    uint4 xr[UN], dyr[UN];
    RowBits<E, GPV * W> wr[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (t + u < t1) {
        xr[u] = ld16nt(xp + (int64_t)(t + u) * D);
        dyr[u] = ld16nt(dyp + (int64_t)(t + u) * D);
        wr[u] = ld_row<E, GPV * W, true>(wp + (int64_t)(t + u) * wstride);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u)
      if (t + u < t1)
        hw_bwd_token<E, W, GPV, ACT, VL>(xp, dyp, wp, dxp, dwp, D, wstride, t + u, t0, t1, T, L,
                                         lane_in_group, rho, win, acc, xr[u], dyr[u], wr[u],
                                         VL ? pos[(int64_t)b * T + t + u] : 0);
  }
  // right halo: tokens t1 .. t1+W-2 complete dx of the chunk's last W-1 tokens
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int t = t1 + j;
    uint4 xr = make_uint4(0, 0, 0, 0), dyr = make_uint4(0, 0, 0, 0);
    RowBits<E, GPV * W> wr = {};
    int p = 0;
    if (t < T) {
      if (ACT) xr = ld16nt(xp + (int64_t)t * D);
      dyr = ld16nt(dyp + (int64_t)t * D);
      wr = ld_row<E, GPV * W, true>(wp + (int64_t)t * wstride);
      if constexpr (VL) p = pos[(int64_t)b * T + t];
    }
    hw_bwd_token<E, W, GPV, ACT, VL>(xp, dyp, wp, dxp, dwp, D, wstride, t, t0, t1, T, L,
                                     lane_in_group, rho, win, acc, xr, dyr, wr, p);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
static int pick_chunk(int T) {
  // long chunks amortise the (W-1)-row halo; 64 tokens keep > 8 waves per CU
  // at the benchmark shapes
  if (T >= 64) return 64;
  return T;
}

template <typename E, int W, int GPV, bool ACT, bool VL>
static hipError_t launch_hw(const HwArgs &a) {
  constexpr int V = Vw<E>::n;
  const int nvec = (int)(a.D / V);
  const int TC = pick_chunk((int)a.T);
  const int nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t G = a.D / a.H;
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  if (!a.bwd) {
    const int nvb = (nvec + kThreads - 1) / kThreads;
    const int64_t nblocks = (int64_t)a.B * nchunk * nvb;
    hipLaunchKernelGGL((hw_fwd_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, s, (const E *)a.x, (const E *)a.w, a.pos, (E *)a.y,
                       (int)a.T, a.D, G, a.H, nvec, nvb, TC, nchunk, rho);
  } else {
    const int L = GPV == 1 ? a.H / V : 1;  // lanes per filter group
    const int U = 64 / L * L;              // lanes of a wave in whole groups
    const int per = U * (kThreads / 64);   // vectors per workgroup
    const int nvb = (nvec + per - 1) / per;
    const int64_t nblocks = (int64_t)a.B * nchunk * nvb;
    hipLaunchKernelGGL((hw_bwd_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(kThreads), 0, s, (const E *)a.x, (const E *)a.w, (const E *)a.dy,
                       a.pos, (E *)a.dx, (E *)a.dw, (int)a.T, a.D, G, a.H, nvec, nvb, TC,
                       nchunk, rho, U);
  }
  return hipGetLastError();
}

template <typename E, int W, int GPV, bool ACT>
static hipError_t dispatch_vl(const HwArgs &a) {
  return a.pos ? launch_hw<E, W, GPV, ACT, true>(a) : launch_hw<E, W, GPV, ACT, false>(a);
}

template <typename E, int W, int GPV>
static hipError_t dispatch_act(const HwArgs &a) {
  return a.act ? dispatch_vl<E, W, GPV, true>(a) : dispatch_vl<E, W, GPV, false>(a);
}

template <typename E, int W>
static hipError_t dispatch_gpv(const HwArgs &a) {
  constexpr int V = Vw<E>::n;
  const int gpv = a.H < V ? V / a.H : 1;
  switch (gpv) {
    case 1: return dispatch_act<E, W, 1>(a);
    case 2: return dispatch_act<E, W, 2>(a);
    case 4: return dispatch_act<E, W, 4>(a);
    default:
      if constexpr (V == 8) return dispatch_act<E, W, 8>(a);
      return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t dispatch_w(const HwArgs &a) {
  switch (a.W) {
    case 1: return dispatch_gpv<E, 1>(a);
    case 2: return dispatch_gpv<E, 2>(a);
    case 3: return dispatch_gpv<E, 3>(a);
    case 4: return dispatch_gpv<E, 4>(a);
    case 5: return dispatch_gpv<E, 5>(a);
    case 6: return dispatch_gpv<E, 6>(a);
    case 7: return dispatch_gpv<E, 7>(a);
    case 8: return dispatch_gpv<E, 8>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t headwise_launch(const HwArgs &a) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  return a.bf16 ? dispatch_w<bf16>(a) : dispatch_w<float>(a);
}

}  // namespace dsc
