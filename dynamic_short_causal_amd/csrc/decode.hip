// decode.hip -- one-token steps of the dynamic short convolution (inference).
//
// Operation: the causal sum of the gist.science summary "Dynamische Korte
// Convoluties Verbeteren Transformers", Methodologie > Dynamische Korte
// Convoluties (bullet Mechanisme; Parametrisatie 1 and 2; Plaatsing, residual),
// evaluated at the newest token t only.  The W-1 previous inputs are kept in a
// state (B, W-1, D), oldest row first:
//   y[b,c] = act(sum_k w[b,g(c),k] x_{t-k}[b,c]) + rho x_t[b,c],
//   x_{t-0} = x_t,  x_{t-k} = state[b, W-1-k, c] (k >= 1),
// after which the state drops its oldest row and appends x_t.  The pages leave
// inference engineering open (wispaper.ai blog "Dynamic Short Convolutions",
// Limitations); this is the plain streaming form of the same sum.
//
// Mapping: a thread owns one 16-byte channel vector of one sequence (head-wise)
// or of a block of sequences (low-rank).  Per sequence it reads x_t, its W-1
// state rows and the filter taps of its groups (head-wise: a row of w;
// low-rank: w = z U formed in registers from R rows of U), writes y and
// rewrites its own slice of the state, so the update in place has a single
// owner.  A decode step is a few FMAs per byte moved, far too little to fill
// matrix cores, so the rank contraction runs on the vector ALUs.
#include "dsc_device.hpp"
#include "decode_launch.hpp"

namespace dsc {

constexpr int kDecThreads = 256;

template <typename E>
__device__ __forceinline__ float to_f32(E v) {
  if constexpr (sizeof(E) == 2) return __uint_as_float((uint32_t)v << 16);
  else return v;
}

// The state update and output of one sequence b for one channel vector c0.
template <typename E, int W, int GPV>
__device__ __forceinline__ void decode_one(const E *__restrict__ x, E *__restrict__ state,
                                           E *__restrict__ y, int64_t b, int64_t D,
                                           int64_t c0, const float (&taps)[GPV * W],
                                           float rho, int act) {
  constexpr int V = Vw<E>::n, S = W - 1, HS = V / GPV;
  const uint4 xraw = ld16(x + b * D + c0);
  float xt[V];
  unpack<E>(xraw, xt);
  uint4 sraw[S > 0 ? S : 1];
  float st[S > 0 ? S : 1][V];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    sraw[j] = ld16(state + (b * S + j) * D + c0);
    unpack<E>(sraw[j], st[j]);
  }
  float o[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int gi = i / HS;
    float s = taps[gi * W] * xt[i];
#pragma unroll
    for (int k = 1; k < W; ++k) s = fmaf(taps[gi * W + k], st[S - k][i], s);
    if (act) s = silu_f(s);
    o[i] = fmaf(rho, xt[i], s);
  }
  st16(y + b * D + c0, pack<E>(o));
  // the state slides by one token; its rows move as raw bits
#pragma unroll
  for (int j = 0; j + 1 < S; ++j) st16(state + (b * S + j) * D + c0, sraw[j + 1]);
  if constexpr (S > 0) st16(state + (b * S + S - 1) * D + c0, xraw);
}

// Head-wise: thread idx owns vector idx % nvec of sequence idx / nvec.
template <typename E, int W, int GPV>
__global__ __launch_bounds__(kDecThreads) void decode_hw_kernel(
    const E *__restrict__ x, const E *__restrict__ w, E *__restrict__ state,
    E *__restrict__ y, int64_t B, int64_t D, int H, int nvec, float rho, int act) {
  constexpr int V = Vw<E>::n, NT = GPV * W;
  const int64_t idx = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
  if (idx >= B * nvec) return;
  const int64_t b = idx / nvec;
  const int64_t c0 = (idx - b * nvec) * V;
  const int64_t G = D / H, g0 = c0 / H;  // first filter group of the vector
  float taps[NT];  // taps[gi * W + k]: tap k of group g0 + gi
  unpack_row<E, NT>(ld_row<E, NT>(w + (b * G + g0) * W), taps);
  decode_one<E, W, GPV>(x, state, y, b, D, c0, taps, rho, act);
}

// Low-rank: thread idx owns vector idx % nvec of the NB sequences from
// NB * (idx / nvec).  Each row chunk of U it loads serves all NB sequences,
// which divides the (cache) reads of U by NB; U is R * G * W elements and is
// read once per sequence block.
template <typename E, int W, int GPV, int NB>
__global__ __launch_bounds__(kDecThreads) void decode_lr_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U,
    E *__restrict__ state, E *__restrict__ y, int64_t B, int64_t D, int H, int R, int nvec,
    float rho, int act) {
  constexpr int V = Vw<E>::n, NT = GPV * W;
  const int64_t nsb = (B + NB - 1) / NB;
  const int64_t idx = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
  if (idx >= nsb * nvec) return;
  const int64_t sb = idx / nvec;
  const int64_t c0 = (idx - sb * nvec) * V;
  const int64_t G = D / H, g0 = c0 / H, GW = G * W, b0 = sb * NB;
  float taps[NB][NT];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) taps[i][j] = 0.f;
  // rows of z past B read row B-1; their taps are discarded below
  int64_t zrow[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) zrow[i] = (b0 + i < B ? b0 + i : B - 1) * R;
  // UNR rows of U in flight at once
  constexpr int UNR = NT <= 32 ? 4 : 2;
  int r = 0;
  for (; r + UNR <= R; r += UNR) {
    RowBits<E, NT> ub[UNR];
    float zr[UNR][NB];
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      ub[q] = ld_row<E, NT>(U + (r + q) * GW + g0 * W);
#pragma unroll
      for (int i = 0; i < NB; ++i) zr[q][i] = to_f32<E>(z[zrow[i] + r + q]);
    }
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      float u[NT];
      unpack_row<E, NT>(ub[q], u);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) taps[i][j] = fmaf(zr[q][i], u[j], taps[i][j]);
    }
  }
  for (; r < R; ++r) {
    float u[NT];
    unpack_row<E, NT>(ld_row<E, NT>(U + r * GW + g0 * W), u);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float zr = to_f32<E>(z[zrow[i] + r]);
#pragma unroll
      for (int j = 0; j < NT; ++j) taps[i][j] = fmaf(zr, u[j], taps[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (b0 + i < B) decode_one<E, W, GPV>(x, state, y, b0 + i, D, c0, taps[i], rho, act);
}

// state[b, j] = x[b, T-(W-1)+j] of a prompt (B, T, D), zero before its start
template <typename E>
__global__ __launch_bounds__(kDecThreads) void decode_state_kernel(
    const E *__restrict__ x, E *__restrict__ state, int64_t B, int64_t T, int64_t D, int S,
    int nvec) {
  constexpr int V = Vw<E>::n;
  const int64_t idx = (int64_t)blockIdx.x * kDecThreads + threadIdx.x;
  if (idx >= B * S * nvec) return;
  const int64_t row = idx / nvec;  // b * S + j
  const int64_t c0 = (idx - row * nvec) * V;
  const int64_t b = row / S, j = row - b * S;
  const int64_t t = T - S + j;
  const uint4 v = t >= 0 ? ld16(x + (b * T + t) * D + c0) : make_uint4(0u, 0u, 0u, 0u);
  st16(state + row * D + c0, v);
}

template <typename E, int W, int GPV, int NB>
static hipError_t launch_dec_lr(const DecArgs &a, int nvec, float rho) {
  const int64_t n = (a.B + NB - 1) / NB * nvec;
  const unsigned grid = (unsigned)((n + kDecThreads - 1) / kDecThreads);
  hipLaunchKernelGGL((decode_lr_kernel<E, W, GPV, NB>), dim3(grid), dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const E *)a.x, (const E *)a.z, (const E *)a.U,
                     (E *)a.state, (E *)a.y, a.B, a.D, a.H, a.R, nvec, rho, a.act ? 1 : 0);
  return hipGetLastError();
}

// Threads of one launch at which the low-rank step blocks sequences: four
// 256-thread workgroups per compute unit before blocking, so the grid still
// covers the chip after it.
constexpr int64_t kDecBlockFrom = 4 * 256 * kDecThreads;

template <typename E, int W, int GPV>
static hipError_t launch_dec(const DecArgs &a) {
  constexpr int V = Vw<E>::n, NT = GPV * W;
  const int nvec = (int)(a.D / V);
  if (a.B == 0) return hipSuccess;
  const float rho = a.residual ? 1.f : 0.f;
  if (a.lowrank) {
    if (a.B * nvec < kDecBlockFrom) return launch_dec_lr<E, W, GPV, 1>(a, nvec, rho);
    return launch_dec_lr<E, W, GPV, (NT <= 32 ? 4 : 2)>(a, nvec, rho);
  }
  const int64_t n = a.B * nvec;
  const unsigned grid = (unsigned)((n + kDecThreads - 1) / kDecThreads);
  hipLaunchKernelGGL((decode_hw_kernel<E, W, GPV>), dim3(grid), dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const E *)a.x, (const E *)a.w, (E *)a.state,
                     (E *)a.y, a.B, a.D, a.H, nvec, rho, a.act ? 1 : 0);
  return hipGetLastError();
}

template <typename E, int W>
static hipError_t dec_gpv(const DecArgs &a) {
  constexpr int V = Vw<E>::n;
  const int gpv = a.H < V ? V / a.H : 1;
  switch (gpv) {
    case 1: return launch_dec<E, W, 1>(a);
    case 2: return launch_dec<E, W, 2>(a);
    case 4: return launch_dec<E, W, 4>(a);
    default:
      if constexpr (V == 8) return launch_dec<E, W, 8>(a);
      return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t dec_w(const DecArgs &a) {
  switch (a.W) {
    case 1: return dec_gpv<E, 1>(a);
    case 2: return dec_gpv<E, 2>(a);
    case 3: return dec_gpv<E, 3>(a);
    case 4: return dec_gpv<E, 4>(a);
    case 5: return dec_gpv<E, 5>(a);
    case 6: return dec_gpv<E, 6>(a);
    case 7: return dec_gpv<E, 7>(a);
    case 8: return dec_gpv<E, 8>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t decode_launch(const DecArgs &a) {
  return a.bf16 ? dec_w<bf16>(a) : dec_w<float>(a);
}

template <typename E>
static hipError_t launch_state(const DecArgs &a) {
  constexpr int V = Vw<E>::n;
  const int S = a.W - 1;
  const int nvec = (int)(a.D / V);
  const int64_t n = a.B * S * nvec;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + kDecThreads - 1) / kDecThreads);
  hipLaunchKernelGGL((decode_state_kernel<E>), dim3(grid), dim3(kDecThreads), 0,
                     (hipStream_t)a.stream, (const E *)a.x, (E *)a.state, a.B, a.T, a.D, S,
                     nvec);
  return hipGetLastError();
}

hipError_t decode_state_launch(const DecArgs &a) {
  return a.bf16 ? launch_state<bf16>(a) : launch_state<float>(a);
}

}  // namespace dsc
