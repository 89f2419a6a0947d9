// headwise.hip -- gfx950 kernels of the head-wise dynamic short convolution.
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (bullets
// Mechanisme, Parametrisatie 2 "head-wise tying", Plaatsing "residual").
// The backward is the derivative of that forward.
//
// Mapping (both kernels): one lane owns one 16-byte vector of channels (8 bf16
// or 4 fp32), so a 64-lane wave covers a 1 KiB column of a token row.  A wave
// owns a chunk of TW consecutive tokens of that column and loads all of them
// at once; the NW waves of a workgroup own consecutive chunks of the same
// column, and workgroups are numbered column-fastest, then chunk group, then
// sequence.  The grid is therefore many rounds of short-lived workgroups that
// sweep the activations in address order.  On MI355X that order streams
// faster than long per-workgroup chunks, which keep every workgroup of the
// grid resident at once and spread the reads in flight over the whole tensor:
// a plain copy-like probe of the forward's bytes took 87 us in that
// geometry against 71 us in row order, and the forward itself went from 92
// to 75 us, the backward from 137 to 122 us, at B=8 T=2048 D=6144 H=16 W=4.
// The rows a wave needs from its neighbours' chunks (the W-1 x rows before it,
// and in the backward the W-1 dy rows after it) pass through LDS; only the
// first and last wave of a workgroup read them from device memory.  The
// causal window and the backward's dx accumulators stay in registers.  Lanes
// of one filter group fetch the same filter row (merged by the cache); when a
// group spans L > 1 lanes the filter gradient is summed across those lanes
// with shuffles, and the backward gives each wave 64 / L whole groups (the
// remaining lanes idle when L is not a power of two).  Every output element
// has one writer.
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

// Tokens per wave (TW) and waves per workgroup (NW): the forward takes 4
// tokens and 8 waves, the backward 8 tokens and 4 waves (the measured best at
// B=8 T=2048 D=6144 H=16 W=4 among 2..16 tokens and 2..16 waves).
template <typename E, int W, int GPV> struct HwTile {
  static constexpr int row_bytes = GPV * W * (int)sizeof(E);
  static constexpr bool small_rows = W <= 4 && row_bytes <= 8;
  static constexpr int FTW = 4, FNW = 8;
  // backward: 8 tokens (>= W-1, so a chunk's halo lies in one neighbour) and
  // 4 waves; small rows are loaded all at once, wide ones 4 tokens at a time
  static constexpr int BTW = 8, BNW = 4, BUN = small_rows ? 8 : 4;
  // waves per SIMD the register budget must allow (wide rows: as the compiler fits)
  static constexpr int BMINW = row_bytes <= 16 ? 2 : 1;
  static constexpr int HR = W > 1 ? W - 1 : 1;  // halo rows
  // x rows of a forward chunk that the following chunks read through LDS
  static constexpr int FS = FTW < HR ? FTW : HR;
};

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
__global__ __launch_bounds__((64 * HwTile<E, W, GPV>::FNW)) void hw_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, const int32_t *__restrict__ pos,
    E *__restrict__ y, int T, int64_t D, int64_t G, int H, int nvec, int ncol, int nchunk,
    float rho) {
  constexpr int V = Vw<E>::n;
  constexpr int TW = HwTile<E, W, GPV>::FTW, NW = HwTile<E, W, GPV>::FNW;
  constexpr int HR = HwTile<E, W, GPV>::HR, S = HwTile<E, W, GPV>::FS;
  __shared__ uint4 xs[NW][S][64];  // the last S x rows of each wave's chunk
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
  const int g0 = (v * V) / H;  // first group of this vector (D < 2^31)
  const E *xp = x + (int64_t)b * T * D + c0;
  E *yp = y + (int64_t)b * T * D + c0;
  const E *wp = w + ((int64_t)b * T * G + g0) * W;
  const int64_t wstride = G * W;

  uint4 xr[TW], hr[HR];
  RowBits<E, GPV * W> wr[TW];
  int pr[VL ? TW : 1];  // document positions (packed rows), fetched with the rows
  if (active) {
#pragma unroll
    for (int u = 0; u < TW; ++u)
      if (t0 + u < t1) {
        xr[u] = ld16nt(xp + (int64_t)(t0 + u) * D);
        wr[u] = ld_row<E, GPV * W, true>(wp + (int64_t)(t0 + u) * wstride);
        if constexpr (VL) pr[u] = pos[(int64_t)b * T + t0 + u];
      }
    // x_{t0-k} from before the workgroup's first chunk (zero before the
    // sequence start); x_{t0-k} lies in the chunk d = ceil(k / TW) waves back
#pragma unroll
    for (int k = 1; k < W; ++k)
      if (wave < (k + TW - 1) / TW)
        hr[k - 1] = t0 - k >= 0 ? ld16nt(xp + (int64_t)(t0 - k) * D) : make_uint4(0u, 0u, 0u, 0u);
    // rows for the following waves (whose chunks exist only if this one is full)
    if (t1 - t0 == TW) {
#pragma unroll
      for (int i = 0; i < S; ++i) xs[wave][i][lane] = xr[TW - S + i];
    }
  }
  __syncthreads();
  if (!active) return;
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int d = (k + TW - 1) / TW;  // offset TW*d - k in that chunk, saved from TW - S on
    if (wave >= d) hr[k - 1] = xs[wave - d][TW * d - k - (TW - S)][lane];
  }
  // win[k] = x_{t-k} while token t is processed; each token first shifts the
  // window by one and then unpacks x_t into win[0]
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
      float taps[GPV * W];
      unpack_row<E, GPV * W>(wr[u], taps);
      if constexpr (VL) mask_taps<W, GPV>(taps, pr[u]);
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
      st16nt(yp + (int64_t)(t0 + u) * D, pack<E>(o));
    }
  }
}

// ---------------------------------------------------------------------------
// Backward: ds = dy act'(s);  dx[tau] = sum_k w[tau+k,g,k] ds[tau+k] + rho dy[tau];
//           dw[t,g,k] = sum_{c in g} ds[t,c] x[t-k,c]
// A lane walks the tokens of its chunk in order.  acc[j] holds the partial dx
// of token t-1-j; token t adds w[t,g,k] ds[t] to token t-k, after which the
// dx of token t-W+1 has every term from tokens up to t (hw_bwd_token hands it
// back).  Tokens after the chunk (t1 .. t1+W-2) only feed dx.
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT, bool VL>
__device__ __forceinline__ void hw_bwd_token(
    const E *xp, const E *dyp, const E *wp, E *dxp, E *dwp, int64_t D,
    int64_t wstride, int t, int t0, int t1, int T, int L, int lane_in_group,
    float rho, float (&win)[W][Geo<E, GPV>::V], float (&acc)[W > 1 ? W - 1 : 1][Geo<E, GPV>::V],
    uint4 xr, uint4 dyr, const RowBits<E, GPV * W> &wr, int p, float (&o)[Geo<E, GPV>::V]) {
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
  // input gradient: token t contributes to tokens t, t-1, ..., t-W+1; o is
  // then dx of token t-W+1 as far as tokens up to t reach it
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
}

// One wave: the tokens t0 .. t1-1 of its chunk.  The dx of its last W-1 tokens
// also needs the terms of the next chunk's first W-1 tokens: the wave that
// owns that chunk leaves them in LDS (the partial dx of the W-1 tokens before
// its chunk), so no token is processed twice; only the last wave of a
// workgroup forms them itself from the next chunk's rows.  With small filter
// rows the wave loads its whole chunk at once and takes its x window from the
// previous wave's rows in LDS; with wide rows it loads 4 tokens at a time and
// reads its window from device memory.
template <typename E, int W, int GPV, bool ACT, bool VL>
__global__ __launch_bounds__((64 * HwTile<E, W, GPV>::BNW), (HwTile<E, W, GPV>::BMINW)) void hw_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ w, const E *__restrict__ dy,
    const int32_t *__restrict__ pos, E *__restrict__ dx, E *__restrict__ dw, int T, int64_t D,
    int64_t G, int H, int nvec, int ncol, int nchunk, float rho, int U) {
  using Tl = HwTile<E, W, GPV>;
  constexpr int V = Vw<E>::n;
  constexpr int TW = Tl::BTW, NW = Tl::BNW, UN = Tl::BUN, HR = Tl::HR;
  constexpr bool kLdsWin = Tl::small_rows;
  static_assert(TW >= W - 1 && TW % UN == 0, "a chunk holds its successor's halo");
  __shared__ uint4 xs[kLdsWin ? NW : 1][HR][64];  // last W-1 x rows of each chunk
  __shared__ float part[NW][HR][V][64];           // partial dx of the W-1 tokens before each chunk
  int bid = blockIdx.x;
  const int col = bid % ncol;
  bid /= ncol;
  const int cgs = (nchunk + NW - 1) / NW;
  const int cg = bid % cgs;
  const int b = bid / cgs;
  // Each wave takes U = 64 / L * L consecutive vectors, whole groups of L
  // lanes (U = 64 when L is a power of two); nvec is a multiple of L, so whole
  // groups retire together and the shuffles never mix active and idle lanes.
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int chunk = cg * NW + wave;
  const int v = col * U + lane;
  const bool active = chunk < nchunk && lane < U && v < nvec;
  const int t0 = chunk * TW;
  const int t1 = min(T, t0 + TW);
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
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

  float win[W][V];
  float acc[HR][V];
#pragma unroll
  for (int j = 0; j < HR; ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[j][i] = 0.f;
  // the dx of token tau = t-W+1 after token t: complete when tau is in the
  // chunk, else the terms for the previous chunk's last tokens
  auto emit = [&](int t, const float (&o)[V]) {
    const int tau = t - (W - 1);
    if (tau >= t0) {
      st16nt(dxp + (int64_t)tau * D, pack<E>(o));
    } else if (wave > 0) {
#pragma unroll
      for (int i = 0; i < V; ++i) part[wave][tau - t0 + HR][i][lane] = o[i];
    }
  };
  auto token = [&](int t, uint4 xr, uint4 dyr, const RowBits<E, GPV * W> &wr, int p) {
    float o[V];
    hw_bwd_token<E, W, GPV, ACT, VL>(xp, dyp, wp, dxp, dwp, D, wstride, t, t0, t1, T, L,
                                     lane_in_group, rho, win, acc, xr, dyr, wr, p, o);
    emit(t, o);
  };
  auto window = [&](const uint4 (&hl)[HR]) {
#pragma unroll
    for (int k = 1; k < W; ++k) unpack<E>(hl[k - 1], win[k - 1]);  // win[k-1] = x_{t0-k}
  };
  uint4 hl[HR];
  if (active && (!kLdsWin || wave == 0)) {
#pragma unroll
    for (int k = 1; k < W; ++k) {
      hl[k - 1] = z4;
      if (t0 - k >= 0) hl[k - 1] = ld16nt(xp + (int64_t)(t0 - k) * D);
    }
  }
  if constexpr (kLdsWin) {
    uint4 xr[TW], dyr[TW];
    RowBits<E, GPV * W> wr[TW];
    int pr[VL ? TW : 1];  // document positions (packed rows), fetched with the rows
    if (active) {
#pragma unroll
      for (int u = 0; u < TW; ++u)
        if (t0 + u < t1) {
          xr[u] = ld16nt(xp + (int64_t)(t0 + u) * D);
          dyr[u] = ld16nt(dyp + (int64_t)(t0 + u) * D);
          wr[u] = ld_row<E, GPV * W, true>(wp + (int64_t)(t0 + u) * wstride);
          if constexpr (VL) pr[u] = pos[(int64_t)b * T + t0 + u];
        }
      if (W > 1 && t1 - t0 == TW) {  // later chunks of this workgroup exist only then
#pragma unroll
        for (int i = 0; i < HR; ++i) xs[wave][i][lane] = xr[TW - HR + i];
      }
    }
    __syncthreads();
    if (active) {
      if (wave > 0) {
#pragma unroll
        for (int k = 1; k < W; ++k) hl[k - 1] = xs[wave - 1][HR - k][lane];
      }
      window(hl);
#pragma unroll
      for (int u = 0; u < TW; ++u)
        if (t0 + u < t1) {
          int p = 0;
          if constexpr (VL) p = pr[u];
          token(t0 + u, xr[u], dyr[u], wr[u], p);
        }
    }
  } else {
    if (active) {
      window(hl);
#pragma nounroll
      for (int g = 0; g < TW; g += UN) {  // a loop: unrolled, both groups' loads are hoisted
        uint4 xr[UN], dyr[UN];
        RowBits<E, GPV * W> wr[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u)
          if (t0 + g + u < t1) {
            xr[u] = ld16nt(xp + (int64_t)(t0 + g + u) * D);
            dyr[u] = ld16nt(dyp + (int64_t)(t0 + g + u) * D);
            wr[u] = ld_row<E, GPV * W, true>(wp + (int64_t)(t0 + g + u) * wstride);
          }
#pragma unroll
        for (int u = 0; u < UN; ++u)
          if (t0 + g + u < t1)
            token(t0 + g + u, xr[u], dyr[u], wr[u], VL ? pos[(int64_t)b * T + t0 + g + u] : 0);
      }
    }
  }
  // The sequence's last chunk: tokens past T add nothing, so W-1 empty steps
  // complete its own dx and hand the previous chunk its remaining terms (a
  // chunk shorter than W-1 tokens holds some of them in acc until then).
  if (W > 1 && active && chunk + 1 == nchunk) {
    const RowBits<E, GPV * W> wz = {};
#pragma unroll
    for (int j = 0; j < W - 1; ++j) token(t1 + j, z4, z4, wz, 0);
  }
  if constexpr (W > 1) {
    __syncthreads();
    if (!active) return;
    if (chunk + 1 < nchunk && wave + 1 < NW) {
      // this chunk is full; the next wave left the terms of its first tokens
#pragma unroll
      for (int j = 0; j < HR; ++j) {
        float o[V];
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = acc[j][i] + part[wave + 1][HR - 1 - j][i][lane];
        st16nt(dxp + (int64_t)(t1 - 1 - j) * D, pack<E>(o));
      }
    } else if (chunk + 1 < nchunk) {
      // the next chunk belongs to another workgroup: take its first W-1 tokens here
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        const int t = t1 + j;
        uint4 xh = z4, dyh = z4;
        RowBits<E, GPV * W> wh = {};
        int p = 0;
        if (t < T) {
          if constexpr (ACT) xh = ld16nt(xp + (int64_t)t * D);
          dyh = ld16nt(dyp + (int64_t)t * D);
          wh = ld_row<E, GPV * W, true>(wp + (int64_t)t * wstride);
          if constexpr (VL) p = pos[(int64_t)b * T + t];
        }
        token(t, xh, dyh, wh, p);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Windows of W = 5..8: long chunks.  Each lane walks TC = 64 tokens of its
// vector with the window in registers, loading 4 tokens ahead; workgroups of 4
// waves cover 256 consecutive vectors of one chunk.  For these windows the
// tall tiles above cost more than their access order saves: the halo of W-1
// rows per chunk and the registers of the wider window (measured at B=4
// T=4096 D=8192 H=64 W=8: forward 110 against 114 us, backward 201 against
// 464 us or more).  In the backward the lane walks t = t0 .. t1+W-2; tokens
// t1 .. t1+W-2 (the right halo) only complete dx of the chunk's last tokens.
// ---------------------------------------------------------------------------
constexpr int kLongThreads = 256;
constexpr int kLongChunk = 64;

template <typename E, int W, int GPV, bool ACT, bool VL>
__global__ __launch_bounds__(kLongThreads) void hw_fwd_long_kernel(
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
  const int v = vb * kLongThreads + threadIdx.x;
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

template <typename E, int W, int GPV, bool ACT, bool VL>
__global__ __launch_bounds__(kLongThreads) void hw_bwd_long_kernel(
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
  const int v = (vb * (kLongThreads / 64) + (int)(threadIdx.x >> 6)) * U + lane;
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
  // token t, then the store of dx of token t-W+1 when it lies in the chunk
  auto long_token = [&](int t, uint4 xr, uint4 dyr, const RowBits<E, GPV * W> &wr, int p) {
    float o[V];
    hw_bwd_token<E, W, GPV, ACT, VL>(xp, dyp, wp, dxp, dwp, D, wstride, t, t0, t1, T, L,
                                     lane_in_group, rho, win, acc, xr, dyr, wr, p, o);
    const int tau = t - (W - 1);
    if (tau >= t0 && tau < t1) st16nt(dxp + (int64_t)tau * D, pack<E>(o));
  };
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
        long_token(t + u, xr[u], dyr[u], wr[u], VL ? pos[(int64_t)b * T + t + u] : 0);
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
    long_token(t, xr, dyr, wr, p);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT, bool VL>
static hipError_t launch_hw_tall(const HwArgs &a) {
  using Tl = HwTile<E, W, GPV>;
  constexpr int V = Vw<E>::n;
  const int nvec = (int)(a.D / V);
  const int64_t G = a.D / a.H;
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  if (!a.bwd) {
    const int nchunk = (int)((a.T + Tl::FTW - 1) / Tl::FTW);
    const int ncol = (nvec + 63) / 64;
    const int64_t nblocks = (int64_t)a.B * ((nchunk + Tl::FNW - 1) / Tl::FNW) * ncol;
    hipLaunchKernelGGL((hw_fwd_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(64 * Tl::FNW), 0, s, (const E *)a.x, (const E *)a.w, a.pos,
                       (E *)a.y, (int)a.T, a.D, G, a.H, nvec, ncol, nchunk, rho);
  } else {
    const int nchunk = (int)((a.T + Tl::BTW - 1) / Tl::BTW);
    const int L = GPV == 1 ? a.H / V : 1;  // lanes per filter group
    const int U = 64 / L * L;              // lanes of a wave in whole groups
    const int ncol = (nvec + U - 1) / U;
    const int64_t nblocks = (int64_t)a.B * ((nchunk + Tl::BNW - 1) / Tl::BNW) * ncol;
    hipLaunchKernelGGL((hw_bwd_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(64 * Tl::BNW), 0, s, (const E *)a.x, (const E *)a.w,
                       (const E *)a.dy, a.pos, (E *)a.dx, (E *)a.dw, (int)a.T, a.D, G, a.H,
                       nvec, ncol, nchunk, rho, U);
  }
  return hipGetLastError();
}

template <typename E, int W, int GPV, bool ACT, bool VL>
static hipError_t launch_hw_long(const HwArgs &a) {
  constexpr int V = Vw<E>::n;
  const int nvec = (int)(a.D / V);
  const int TC = a.T < kLongChunk ? (int)a.T : kLongChunk;
  const int nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t G = a.D / a.H;
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  if (!a.bwd) {
    const int nvb = (nvec + kLongThreads - 1) / kLongThreads;
    const int64_t nblocks = (int64_t)a.B * nchunk * nvb;
    hipLaunchKernelGGL((hw_fwd_long_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(kLongThreads), 0, s, (const E *)a.x, (const E *)a.w, a.pos,
                       (E *)a.y, (int)a.T, a.D, G, a.H, nvec, nvb, TC, nchunk, rho);
  } else {
    const int L = GPV == 1 ? a.H / V : 1;  // lanes per filter group
    const int U = 64 / L * L;              // lanes of a wave in whole groups
    const int per = U * (kLongThreads / 64);   // vectors per workgroup
    const int nvb = (nvec + per - 1) / per;
    const int64_t nblocks = (int64_t)a.B * nchunk * nvb;
    hipLaunchKernelGGL((hw_bwd_long_kernel<E, W, GPV, ACT, VL>), dim3((unsigned)nblocks),
                       dim3(kLongThreads), 0, s, (const E *)a.x, (const E *)a.w,
                       (const E *)a.dy, a.pos, (E *)a.dx, (E *)a.dw, (int)a.T, a.D, G, a.H,
                       nvec, nvb, TC, nchunk, rho, U);
  }
  return hipGetLastError();
}

template <typename E, int W, int GPV, bool ACT, bool VL>
static hipError_t launch_hw(const HwArgs &a) {
  if constexpr (W <= 4) return launch_hw_tall<E, W, GPV, ACT, VL>(a);
  else return launch_hw_long<E, W, GPV, ACT, VL>(a);
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
