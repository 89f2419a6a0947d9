// static.hip -- gfx950 kernels of the static short convolution: one causal
// filter per group, the same for every sequence and position.
//
// Operation: the causal sum y_t = sum_k w_k x_{t-k} with a fixed w
// (wispaper.ai blog "Dynamic Short Convolutions", Methodology > 1.
// Mathematical Intuition; the digg.com thread calls it a depthwise-separable
// causal convolution of small width), with the head-wise tying, residual and
// SiLU of the dynamic path.  It is the yardstick the pages measure the
// dynamic kernels against (gist.science summary, Efficiente
// Trainingsimplementatie, bullet Prestaties).  The backward is the derivative.
//
// Forward mapping: one lane owns one 16-byte channel vector with the causal
// window in registers, in the head-wise forward's layouts (short chunks in
// address order for W <= 4, long strips above), but its filter taps are
// loaded once and kept in registers, so the kernel streams only x in and y
// out.
//
// Backward mapping: a workgroup of kStWaves waves owns 64 channel vectors;
// wave i walks chunk kStWaves * cg + i of them.  dx is formed as in the
// head-wise backward.  dw, summed over every token, accumulates in registers
// over the lane's chunk, then over the L lanes of a group that spans several
// vectors (shuffles), then over the waves (LDS, fixed order).  One fp32 row of
// G * W per (sequence, chunk group) goes to the workspace, and a second kernel
// adds the rows in ascending order, so dw is bitwise reproducible.
#include "dsc_device.hpp"
#include "static_launch.hpp"

namespace dsc {

constexpr int kStFwdThreads = 256;
constexpr int kStBwdThreads = 64 * kStWaves;
constexpr int kStRedThreads = 256;

// ---------------------------------------------------------------------------
// Forward: y[t] = act(sum_k w[g,k] x[t-k]) + rho x[t]
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT>
__global__ __launch_bounds__(kStFwdThreads) void st_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, E *__restrict__ y, int T, int64_t D,
    int H, int nvec, int nvb, int TC, int nchunk, float rho) {
  constexpr int V = Vw<E>::n, HS = V / GPV, NT = GPV * W;
  constexpr int UN = 4;  // tokens loaded ahead per step
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int v = vb * kStFwdThreads + threadIdx.x;
  if (v >= nvec) return;
  const int t0 = chunk * TC;
  const int t1 = min(T, t0 + TC);
  const int64_t c0 = (int64_t)v * V;
  const E *xp = x + (int64_t)b * T * D + c0;
  E *yp = y + (int64_t)b * T * D + c0;
  float taps[NT];
  unpack_row<E, NT>(ld_row<E, NT>(w + (c0 / H) * W), taps);

  // win[k] = x_{t-k} while token t is processed (zero before the sequence)
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
#pragma unroll
    for (int u = 0; u < UN; ++u)
      if (t + u < t1) xr[u] = ld16nt(xp + (int64_t)(t + u) * D);
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (t + u < t1) {
#pragma unroll
        for (int k = W - 1; k > 0; --k)
#pragma unroll
          for (int i = 0; i < V; ++i) win[k][i] = win[k - 1][i];
        unpack<E>(xr[u], win[0]);
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int gi = i / HS;
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

// Forward for W <= 4 in the head-wise forward's short-chunk order: a wave
// takes 4 consecutive tokens of one 64-vector column, loaded at once; the 8
// waves of a workgroup take consecutive chunks of that column; workgroups run
// column-fastest.  The x rows before a chunk come from the previous wave
// through LDS (the first wave of a workgroup reads them from memory).
constexpr int kStTallTW = 4, kStTallNW = 8;
template <typename E, int W, int GPV, bool ACT>
__global__ __launch_bounds__(64 * kStTallNW) void st_fwd_tall_kernel(
    const E *__restrict__ x, const E *__restrict__ w, E *__restrict__ y, int T, int64_t D,
    int H, int nvec, int ncol, int nchunk, float rho) {
  constexpr int V = Vw<E>::n, HS = V / GPV, NT = GPV * W;
  constexpr int TW = kStTallTW, NW = kStTallNW, HR = W > 1 ? W - 1 : 1;
  static_assert(TW >= W - 1, "the window lies in the previous chunk");
  __shared__ uint4 xs[NW][HR][64];  // the last W-1 x rows of each wave's chunk
  int bid = blockIdx.x;
  const int col = bid % ncol;
  bid /= ncol;
  const int cgs = (nchunk + NW - 1) / NW;
  const int cg = bid % cgs;
  const int b = bid / cgs;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int chunk = cg * NW + wave;
  const int v = col * 64 + lane;
  const bool active = chunk < nchunk && v < nvec;
  const int t0 = chunk * TW;
  const int t1 = min(T, t0 + TW);
  const int64_t c0 = (int64_t)v * V;
  const E *xp = x + (int64_t)b * T * D + c0;
  E *yp = y + (int64_t)b * T * D + c0;
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  uint4 xr[TW], hr[HR];
  float taps[NT];
  if (active) {
#pragma unroll
    for (int u = 0; u < TW; ++u)
      if (t0 + u < t1) xr[u] = ld16nt(xp + (int64_t)(t0 + u) * D);
    unpack_row<E, NT>(ld_row<E, NT>(w + (c0 / H) * W), taps);
    if (wave == 0) {
#pragma unroll
      for (int k = 1; k < W; ++k) {
        hr[k - 1] = z4;
        if (t0 - k >= 0) hr[k - 1] = ld16nt(xp + (int64_t)(t0 - k) * D);
      }
    }
    if (W > 1 && t1 - t0 == TW) {  // later chunks of this workgroup exist only then
#pragma unroll
      for (int i = 0; i < HR; ++i) xs[wave][i][lane] = xr[TW - HR + i];
    }
  }
  __syncthreads();
  if (!active) return;
  if (wave > 0) {
#pragma unroll
    for (int k = 1; k < W; ++k) hr[k - 1] = xs[wave - 1][HR - k][lane];
  }
  // win[k] = x_{t-k} while token t is processed
  float win[W][V];
#pragma unroll
  for (int k = 1; k < W; ++k) unpack<E>(hr[k - 1], win[k - 1]);
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    if (t0 + u < t1) {
#pragma unroll
      for (int k = W - 1; k > 0; --k)
#pragma unroll
        for (int i = 0; i < V; ++i) win[k][i] = win[k - 1][i];
      unpack<E>(xr[u], win[0]);
      float o[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int gi = i / HS;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) s = fmaf(taps[gi * W + k], win[k][i], s);
        if constexpr (ACT) s = silu_f(s);
        o[i] = fmaf(rho, win[0][i], s);
      }
      st16nt(yp + (int64_t)(t0 + u) * D, pack<E>(o));
    }
  }
}

// ---------------------------------------------------------------------------
// Backward.  The lane walks t = t0 .. t1+W-2; acc[j] holds the partial dx of
// token t-1-j.  Token t adds w[g,k] ds[t] to token t-k, after which token
// t-W+1 is complete and is stored.  Tokens t1 .. t1+W-2 (the right halo) only
// feed dx; tokens of the chunk also add ds[t] x[t-k] to dw.
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT>
__device__ __forceinline__ void st_bwd_token(
    E *dxp, int64_t D, int t, int t0, int t1, int T, float rho, const float (&taps)[GPV * W],
    float (&win)[W][Vw<E>::n], float (&acc)[W > 1 ? W - 1 : 1][Vw<E>::n],
    float (&dwa)[GPV * W], uint4 xr, uint4 dyr) {
  constexpr int V = Vw<E>::n, HS = V / GPV;
  const bool in_chunk = t < t1;
#pragma unroll
  for (int k = W - 1; k > 0; --k)
#pragma unroll
    for (int i = 0; i < V; ++i) win[k][i] = win[k - 1][i];
  float dyv[V], ds[V];
  if (t < T) {
    unpack<E>(dyr, dyv);
    if (ACT || in_chunk) {
      unpack<E>(xr, win[0]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) win[0][i] = 0.f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) { dyv[i] = 0.f; win[0][i] = 0.f; }
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
  if (in_chunk) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int gi = i / HS;
#pragma unroll
      for (int k = 0; k < W; ++k) dwa[gi * W + k] = fmaf(ds[i], win[k][i], dwa[gi * W + k]);
    }
  }
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

template <typename E, int W, int GPV, bool ACT>
__global__ __launch_bounds__(kStBwdThreads) void st_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, const E *__restrict__ dy,
    E *__restrict__ dx, float *__restrict__ part, int T, int64_t D, int H, int nvec,
    int nvb, int TC, int ncg, float rho, int U) {
  constexpr int V = Vw<E>::n, NT = GPV * W;
  constexpr int UN = 4;
  __shared__ float red[kStWaves][NT][64];
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int cg = bid % ncg;
  const int b = bid / ncg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // the workgroup's waves share U = 64 / L * L vectors, whole groups of L
  // lanes; lanes past U or past D only join the barrier
  const int v = vb * U + lane;
  const bool active = lane < U && v < nvec;
  const int t0 = min(T, (cg * kStWaves + wave) * TC);
  const int t1 = min(T, t0 + TC);
  const int64_t c0 = (int64_t)(active ? v : 0) * V;
  const int64_t G = D / H;
  const int g0 = (int)(c0 / H);
  const int L = (GPV == 1) ? H / V : 1;  // lanes sharing one group (aligned)

  float dwa[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) dwa[j] = 0.f;
  if (active && t0 < t1) {
    const int64_t base = (int64_t)b * T * D + c0;
    const E *xp = x + base;
    const E *dyp = dy + base;
    E *dxp = dx + base;
    float taps[NT];
    unpack_row<E, NT>(ld_row<E, NT>(w + (int64_t)g0 * W), taps);
    float win[W][V];
    float acc[W > 1 ? W - 1 : 1][V];
#pragma unroll
    for (int j = 0; j < (W > 1 ? W - 1 : 1); ++j)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[j][i] = 0.f;
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
      uint4 xr[UN], dyr[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        if (t + u < t1) {
          xr[u] = ld16nt(xp + (int64_t)(t + u) * D);
          dyr[u] = ld16nt(dyp + (int64_t)(t + u) * D);
        }
      }
#pragma unroll
      for (int u = 0; u < UN; ++u)
        if (t + u < t1)
          st_bwd_token<E, W, GPV, ACT>(dxp, D, t + u, t0, t1, T, rho, taps, win, acc, dwa,
                                       xr[u], dyr[u]);
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int t = t1 + j;
      uint4 xr = make_uint4(0, 0, 0, 0), dyr = make_uint4(0, 0, 0, 0);
      if (t < T) {
        if (ACT) xr = ld16nt(xp + (int64_t)t * D);
        dyr = ld16nt(dyp + (int64_t)t * D);
      }
      st_bwd_token<E, W, GPV, ACT>(dxp, D, t, t0, t1, T, rho, taps, win, acc, dwa, xr, dyr);
    }
  }
  // sum over the L lanes of a group: aligned runs of L lanes inside the wave,
  // all active or all idle since nvec % L == 0
  if constexpr (GPV == 1) group_sum<W>(dwa, L, lane % L);
#pragma unroll
  for (int j = 0; j < NT; ++j) red[wave][j][lane] = dwa[j];
  __syncthreads();
  if (wave == 0 && active && (GPV > 1 || lane % L == 0)) {
    float s[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      s[j] = red[0][j][lane];
#pragma unroll
      for (int i = 1; i < kStWaves; ++i) s[j] += red[i][j][lane];
    }
    float *pp = part + ((int64_t)b * ncg + cg) * G * W + (int64_t)g0 * W;
#pragma unroll
    for (int j = 0; j < NT; ++j) pp[j] = s[j];
  }
}

// dw[j] = sum_{p < parts} part[p][j], in ascending p; zero when parts == 0
template <typename E>
__global__ __launch_bounds__(kStRedThreads) void st_reduce_kernel(
    const float *__restrict__ part, E *__restrict__ dw, int64_t GW, int64_t parts) {
  const int64_t j = (int64_t)blockIdx.x * kStRedThreads + threadIdx.x;
  if (j >= GW) return;
  float s = 0.f;
  int64_t p = 0;
  for (; p + 4 <= parts; p += 4) {
    const float a0 = part[p * GW + j], a1 = part[(p + 1) * GW + j];
    const float a2 = part[(p + 2) * GW + j], a3 = part[(p + 3) * GW + j];
    s += a0; s += a1; s += a2; s += a3;
  }
  for (; p < parts; ++p) s += part[p * GW + j];
  if constexpr (sizeof(E) == 2) {
    dw[j] = (E)(pack_bf16x2(s, 0.f) & 0xffffu);
  } else {
    dw[j] = s;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT>
static hipError_t launch_st(const StArgs &a) {
  constexpr int V = Vw<E>::n;
  const int nvec = (int)(a.D / V);
  const int64_t G = a.D / a.H;
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  const StPlan p = st_plan(a.B, a.T, a.D, a.W, a.H);
  if (!a.bwd) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    if constexpr (W <= 4) {
      const int nchunk = (int)((a.T + kStTallTW - 1) / kStTallTW);
      const int ncol = (nvec + 63) / 64;
      const int64_t nblocks = a.B * ((nchunk + kStTallNW - 1) / kStTallNW) * ncol;
      hipLaunchKernelGGL((st_fwd_tall_kernel<E, W, GPV, ACT>), dim3((unsigned)nblocks),
                         dim3(64 * kStTallNW), 0, s, (const E *)a.x, (const E *)a.w, (E *)a.y,
                         (int)a.T, a.D, a.H, nvec, ncol, nchunk, rho);
      return hipGetLastError();
    }
    const int tc = a.T < kStFwdChunk ? (int)a.T : kStFwdChunk;
    const int nchunk = (int)((a.T + tc - 1) / tc);
    const int nvb = (nvec + kStFwdThreads - 1) / kStFwdThreads;
    const int64_t nblocks = a.B * nchunk * nvb;
    hipLaunchKernelGGL((st_fwd_kernel<E, W, GPV, ACT>), dim3((unsigned)nblocks),
                       dim3(kStFwdThreads), 0, s, (const E *)a.x, (const E *)a.w, (E *)a.y,
                       (int)a.T, a.D, a.H, nvec, nvb, tc, nchunk, rho);
    return hipGetLastError();
  }
  if (a.B > 0 && a.T > 0) {
    const int L = GPV == 1 ? a.H / V : 1;  // lanes per filter group
    const int U = 64 / L * L;              // vectors per workgroup, whole groups
    const int nvb = (nvec + U - 1) / U;
    const int64_t nblocks = a.B * p.ncg * nvb;
    hipLaunchKernelGGL((st_bwd_kernel<E, W, GPV, ACT>), dim3((unsigned)nblocks),
                       dim3(kStBwdThreads), 0, s, (const E *)a.x, (const E *)a.w,
                       (const E *)a.dy, (E *)a.dx, (float *)a.ws, (int)a.T, a.D, a.H, nvec,
                       nvb, p.tc, p.ncg, rho, U);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t GW = G * a.W;
  const unsigned rgrid = (unsigned)((GW + kStRedThreads - 1) / kStRedThreads);
  hipLaunchKernelGGL((st_reduce_kernel<E>), dim3(rgrid), dim3(kStRedThreads), 0, s,
                     (const float *)a.ws, (E *)a.dw, GW,
                     (a.B > 0 && a.T > 0) ? p.parts : (int64_t)0);
  return hipGetLastError();
}

template <typename E, int W, int GPV>
static hipError_t st_act(const StArgs &a) {
  return a.act ? launch_st<E, W, GPV, true>(a) : launch_st<E, W, GPV, false>(a);
}

template <typename E, int W>
static hipError_t st_gpv(const StArgs &a) {
  constexpr int V = Vw<E>::n;
  const int gpv = a.H < V ? V / a.H : 1;
  switch (gpv) {
    case 1: return st_act<E, W, 1>(a);
    case 2: return st_act<E, W, 2>(a);
    case 4: return st_act<E, W, 4>(a);
    default:
      if constexpr (V == 8) return st_act<E, W, 8>(a);
      return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t st_w(const StArgs &a) {
  switch (a.W) {
    case 1: return st_gpv<E, 1>(a);
    case 2: return st_gpv<E, 2>(a);
    case 3: return st_gpv<E, 3>(a);
    case 4: return st_gpv<E, 4>(a);
    case 5: return st_gpv<E, 5>(a);
    case 6: return st_gpv<E, 6>(a);
    case 7: return st_gpv<E, 7>(a);
    case 8: return st_gpv<E, 8>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t static_launch(const StArgs &a) {
  return a.bf16 ? st_w<bf16>(a) : st_w<float>(a);
}

}  // namespace dsc
