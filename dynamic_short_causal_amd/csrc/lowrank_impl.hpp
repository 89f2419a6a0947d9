// lowrank_impl.hpp -- gfx950 kernels of the low-rank dynamic short convolution.
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (Mechanisme;
// Parametrisatie 1, low-rank factorisation of rank R; Plaatsing, residual)
// and Efficiente Trainingsimplementatie, bullet "Fused Low-Rank Kernel": the
// filters w[t,g,k] = sum_r z[t,r] U[r, g*W+k] are produced on chip and used at
// once; they never reach device memory.  The backward is the derivative.
//
// Work decomposition.  A workgroup (4 waves) owns a block of CB channels and a
// chunk of tokens of one sequence; each wave owns CW = 4*NU*V channels.  The
// wave walks its chunk in tiles of 16 tokens.  Inside a tile, lane (q, j)
// (q = lane / 16, j = lane % 16) handles token t+j and the NU channel vectors
// u*4 + q of the wave's slice, so one wave instruction touches 16 token rows
// at 4 adjacent 16-byte vectors.
//
// Filters on chip: for every tap k the wave issues 16x16 MFMAs whose B operand
// is z^T of the 16 tokens (K = ranks) and whose A operand holds the U columns
// of the (group, tap) slots the lanes need.  The output layout of a 16x16
// MFMA gives lane (q, j) rows 4q..4q+3 of column j, so each lane receives
// exactly the filter taps of its own token and channels; the tap sum of the
// convolution then stays in-lane.  bf16 uses v_mfma_f32_16x16x16_bf16 (bf16
// products, fp32 sums); fp32 uses v_mfma_f32_16x16x4_f32.
//
// Backward per tile:
//   * ds = dy (or dy * SiLU'(s), with s recomputed in-lane);
//   * dx[t] = rho dy[t] + sum_k w[t+k,k] ds[t+k]: the products p_k = w_k ds
//     are formed at token t+k and moved k lanes down the 16-lane row with DPP
//     row shifts; the last W-1 tokens of a tile receive their share from the
//     next tile (a one-tile lag), the chunk's last tile from a halo tile;
//   * dw (on chip only) -> dz^T += U dw^T with 16x16x32 bf16 MFMAs (K = the
//     lane's slots), summed across the 4 waves in LDS and written as one fp32
//     partial per channel block;
//   * dU^T += dw^T z: dw is transposed through LDS so tokens become the K
//     dimension; accumulated over the whole chunk in registers and written
//     once per chunk as an fp32 partial.
// A second kernel adds the partials in a fixed order (deterministic).
#pragma once
#include <type_traits>
#include "dsc_device.hpp"
#include "dsc_launch.hpp"

namespace dsc {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLrThreads = 256;

template <typename E, int W, int GPV> struct LrGeo {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int V = Vw<E>::n;
  static constexpr int H = V / GPV;         // channels per filter group
  // channel vectors per lane: up to 4, fewer for wide filters (register budget)
  static constexpr int NUMAX = W <= 3 ? 4 : W <= 6 ? 2 : 1;
  static constexpr int NU = H < NUMAX ? H : NUMAX;
  static constexpr int NG = NU * GPV;       // (group, vector) instances per lane per tap
  static constexpr int NP = (NG + 3) / 4;   // filter MFMAs per tap (4 rows per lane each)
  static constexpr int NS = NG * W;         // filter slots per lane
  static constexpr int CW = 4 * NU * V;     // channels per wave
  static constexpr int CB = 4 * CW;         // channels per workgroup
};

// ---- small helpers -----------------------------------------------------------
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return __uint_as_float((uint32_t)v << 16); }

template <bool BF> struct WFrag { typedef s16x4 T; };
template <> struct WFrag<false> { typedef float T; };
template <bool BF> struct DzFrag { typedef bf16x8_t T; };
template <> struct DzFrag<false> { typedef float T; };

// filter-generation MFMA: 16x16 output, K = 16 (bf16) or 4 (fp32) ranks
template <bool BF>
__device__ __forceinline__ f32x4 mma_w(typename WFrag<BF>::T a, typename WFrag<BF>::T b, f32x4 c) {
  if constexpr (BF) return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// dz MFMA: K = 32 (bf16) or 4 (fp32) filter slots
template <bool BF>
__device__ __forceinline__ f32x4 mma_dz(typename DzFrag<BF>::T a, typename DzFrag<BF>::T b, f32x4 c) {
  if constexpr (BF) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// DPP row shifts inside each 16-lane row, with 0 where the source lane falls
// outside the row.  k is a compile-time constant after unrolling.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// lane l <- lane l+k
__device__ __forceinline__ uint32_t row_shl_u32(uint32_t v, int k) {
  switch (k) {
    case 1: return dpp_u32<0x101>(v);  case 2: return dpp_u32<0x102>(v);
    case 3: return dpp_u32<0x103>(v);  case 4: return dpp_u32<0x104>(v);
    case 5: return dpp_u32<0x105>(v);  case 6: return dpp_u32<0x106>(v);
    case 7: return dpp_u32<0x107>(v);  case 8: return dpp_u32<0x108>(v);
    case 9: return dpp_u32<0x109>(v);  case 10: return dpp_u32<0x10A>(v);
    case 11: return dpp_u32<0x10B>(v); case 12: return dpp_u32<0x10C>(v);
    case 13: return dpp_u32<0x10D>(v); case 14: return dpp_u32<0x10E>(v);
    case 15: return dpp_u32<0x10F>(v); default: return v;
  }
}
// lane l <- lane l-k
__device__ __forceinline__ uint32_t row_shr_u32(uint32_t v, int k) {
  switch (k) {
    case 1: return dpp_u32<0x111>(v);  case 2: return dpp_u32<0x112>(v);
    case 3: return dpp_u32<0x113>(v);  case 4: return dpp_u32<0x114>(v);
    case 5: return dpp_u32<0x115>(v);  case 6: return dpp_u32<0x116>(v);
    case 7: return dpp_u32<0x117>(v);  case 8: return dpp_u32<0x118>(v);
    case 9: return dpp_u32<0x119>(v);  case 10: return dpp_u32<0x11A>(v);
    case 11: return dpp_u32<0x11B>(v); case 12: return dpp_u32<0x11C>(v);
    case 13: return dpp_u32<0x11D>(v); case 14: return dpp_u32<0x11E>(v);
    case 15: return dpp_u32<0x11F>(v); default: return v;
  }
}
__device__ __forceinline__ float row_shl(float v, int k) {
  return __uint_as_float(row_shl_u32(__float_as_uint(v), k));
}
// lanes 16-k..15 receive lanes 0..k-1 (row shift right by 16-k)
__device__ __forceinline__ float row_shr_16mk(float v, int k) {
  return __uint_as_float(row_shr_u32(__float_as_uint(v), 16 - k));
}
// Tap k of a 16-token tile held one token per lane: lane j gets the vector of
// token t+j-k, from lane j-k of this tile or lane 16-k+j of the previous one.
__device__ __forceinline__ uint4 tap_vec(uint4 cur, uint4 prev, int k) {
  if (k == 0) return cur;
  return make_uint4(row_shr_u32(cur.x, k) | row_shl_u32(prev.x, 16 - k),
                    row_shr_u32(cur.y, k) | row_shl_u32(prev.y, 16 - k),
                    row_shr_u32(cur.z, k) | row_shl_u32(prev.z, 16 - k),
                    row_shr_u32(cur.w, k) | row_shl_u32(prev.w, 16 - k));
}
__device__ __forceinline__ uint4 sel4(bool ok, uint4 v) {
  return ok ? v : make_uint4(0u, 0u, 0u, 0u);
}

// Filter slot sigma = k*NG + m of lane quarter qq; m = u*GPV + gi names vector
// u*4 + qq of the wave slice and group gi inside it.  Returns the U column,
// or -1 when the channel lies beyond D.
template <typename E, int W, int GPV>
__device__ __forceinline__ int slot_col(int cw, int qq, int k, int m, int D) {
  using Gm = LrGeo<E, W, GPV>;
  const int u = m / GPV, gi = m % GPV;
  const int c = cw + (u * 4 + qq) * Gm::V;
  if (c >= D) return -1;
  return (c / Gm::H + gi) * W + k;
}

// A operands of the filter MFMAs: for tap k, part p, rank step ks, lane (qa, i)
// holds U[ranks of K-quarter qa][column of output row i].
template <typename E, int W, int GPV, int KS>
__device__ __forceinline__ void load_wA(const E *__restrict__ U, int GW, int R, int cw, int D,
                                        int lane,
                                        typename WFrag<sizeof(E) == 2>::T (&a)[W][LrGeo<E, W, GPV>::NP][KS]) {
  using Gm = LrGeo<E, W, GPV>;
  const int qa = lane >> 4, i = lane & 15, qo = i >> 2, e = i & 3;
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int p = 0; p < Gm::NP; ++p) {
      const int m = 4 * p + e;
      const int col = m < Gm::NG ? slot_col<E, W, GPV>(cw, qo, k, m, D) : -1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (Gm::BF) {
          s16x4 f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = ks * 16 + 4 * qa + e2;
            f[e2] = (col >= 0 && r < R) ? (short)U[(int64_t)r * GW + col] : (short)0;
          }
          a[k][p][ks] = f;
        } else {
          const int r = ks * 4 + qa;
          a[k][p][ks] = (col >= 0 && r < R) ? (float)U[(int64_t)r * GW + col] : 0.f;
        }
      }
    }
}

// B operand of the filter MFMAs: z^T of token `tok` (lane (q, j) holds ranks
// of K-quarter q).  Branch-free so it can be issued a tile ahead: a lane with
// no token (`valid` false) reads the first z row instead.  Such lanes' filters
// are never used for an output, and ranks r >= R meet zero rows of U, so the
// fragment needs no masking.
template <typename E, int KS>
__device__ __forceinline__ void load_zB(const E *__restrict__ z, int64_t tok, bool valid, int R,
                                        int q, typename WFrag<sizeof(E) == 2>::T (&bz)[KS]) {
  constexpr bool BF = sizeof(E) == 2;
  const E *zr = z + (valid ? tok * R : 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (BF) {
      const int r0 = ks * 16 + 4 * q;
      s16x4 f;
      if ((R & 3) == 0) {  // 8-byte aligned 4-rank groups, all in or all out
        const uint2 v = *reinterpret_cast<const uint2 *>(r0 < R ? zr + r0 : z);
        f[0] = (short)(v.x & 0xffff); f[1] = (short)(v.x >> 16);
        f[2] = (short)(v.y & 0xffff); f[3] = (short)(v.y >> 16);
      } else {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) f[e2] = (short)(r0 + e2 < R ? zr[r0 + e2] : z[0]);
      }
      bz[ks] = f;
    } else {
      const int r = ks * 4 + q;
      bz[ks] = r < R ? zr[r] : z[0];
    }
  }
}

// Filters of the 16 tokens of a tile: acc[k][p][e] at lane (q, j) is the tap-k
// weight of slot m = 4p+e of token t+j.
template <typename E, int W, int GPV, int KS>
__device__ __forceinline__ void gen_filters(
    const typename WFrag<sizeof(E) == 2>::T (&a)[W][LrGeo<E, W, GPV>::NP][KS],
    const typename WFrag<sizeof(E) == 2>::T (&bz)[KS], f32x4 (&acc)[W][LrGeo<E, W, GPV>::NP]) {
  using Gm = LrGeo<E, W, GPV>;
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int p = 0; p < Gm::NP; ++p) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) c = mma_w<Gm::BF>(a[k][p][ks], bz[ks], c);
      acc[k][p] = c;
    }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, bool ACT, int RB>
__global__ __launch_bounds__(kLrThreads) void lr_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U, E *__restrict__ y,
    int T, int D, int R, int TC, int nchunk, int ncb, float rho) {
  using Gm = LrGeo<E, W, GPV>;
  constexpr int V = Gm::V, NU = Gm::NU, NP = Gm::NP;
  constexpr int KS = RB * (Gm::BF ? 1 : 4);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, j = lane & 15;
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int cw = cb * Gm::CB + wave * Gm::CW;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int GW = (D / Gm::H) * W;

  typename WFrag<Gm::BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV, KS>(U, GW, R, cw, D, lane, aw);

  const int64_t seq = (int64_t)b * T;
  // Each lane loads only the x row of its own token (one 16-byte vector per
  // unit); taps k >= 1 come from the neighbouring lanes by DPP (tap_vec), the
  // first W-1 lanes of a tile from the previous tile's registers.  Loads are
  // issued one tile ahead and are branch-free: a lane without a token or
  // channel reads row 0 and zeroes it on use.
  typename WFrag<Gm::BF>::T zn[KS];
  uint4 xn[NU], xp[NU];
  auto issue = [&](int t) {
    const int tau = t + j;
    const bool valid = tau < t1;
    load_zB<E, KS>(z, seq + tau, valid, R, q, zn);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = cw + (u * 4 + q) * V;
      xn[u] = ld16(x + (valid && c < D ? (seq + tau) * D + c : 0));
    }
  };
  // the 16 tokens before the chunk (zero before the sequence start)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = cw + (u * 4 + q) * V;
    const int tb = t0 - 16 + j;
    const bool ok = tb >= 0 && c < D;
    xp[u] = sel4(ok, ld16(x + (ok ? (seq + tb) * D + c : 0)));
  }
  issue(t0);
  for (int t = t0; t < t1; t += 16) {
    const int tau = t + j;
    const bool valid = tau < t1;
    typename WFrag<Gm::BF>::T bz[KS];
    uint4 xc[NU];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bz[ks] = zn[ks];
#pragma unroll
    for (int u = 0; u < NU; ++u) xc[u] = sel4(valid && cw + (u * 4 + q) * V < D, xn[u]);
    if (t + 16 < t1) issue(t + 16);  // wave-uniform
    f32x4 wacc[W][NP];
    gen_filters<E, W, GPV, KS>(aw, bz, wacc);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = cw + (u * 4 + q) * V;
      float xk[W][V];
#pragma unroll
      for (int k = 0; k < W; ++k) unpack<E>(tap_vec(xc[u], xp[u], k), xk[k]);
      float o[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int m = u * GPV + i / Gm::H;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) s = fmaf(wacc[k][m >> 2][m & 3], xk[k][i], s);
        if constexpr (ACT) s = silu_f(s);
        o[i] = fmaf(rho, xk[0][i], s);
      }
      if (valid && c < D) st16(y + (seq + tau) * D + c, pack<E>(o));
      xp[u] = xc[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV, int RB> struct LrBwdSmem {
  using Gm = LrGeo<E, W, GPV>;
  // per wave: dw^T, 4*NS slot rows x 16 tokens, padded with zero rows to
  // whole 16-row MFMA blocks
  static constexpr int nrb = (Gm::NS + 3) / 4;
  static constexpr int dwt_bytes = 16 * nrb * 16 * (int)sizeof(E);
  // per workgroup: two buffers of the 4 waves' dz^T tiles (RB x 64 lanes x 4)
  static constexpr int dz_floats = 2 * 4 * RB * 64 * 4;
  static constexpr int bytes = 4 * dwt_bytes + dz_floats * 4;
};

// Two waves per SIMD (at most 256 VGPR+AGPR per lane) where the compiler fits
// that without spilling, one otherwise.  The set was read off the kernel
// resource-usage report of every instance.
template <typename E, int W, int GPV>
constexpr int lr_bwd_min_waves() {
  if constexpr (sizeof(E) == 2) {
    const bool two = W == 1 || ((W == 2 || W == 3) && GPV == 4) ||
                     (W == 4 && (GPV == 1 || GPV == 8)) || (W == 5 && GPV == 8) ||
                     (W == 7 && (GPV == 1 || GPV == 2));
    return two ? 2 : 1;
  } else {
    const bool two = W <= 4 || (W == 5 && (GPV == 1 || GPV == 4)) ||
                     (W == 7 && (GPV == 1 || GPV == 2)) || (W == 8 && GPV == 1);
    return two ? 2 : 1;
  }
}

template <typename E, int W, int GPV, int RB>
__global__ __launch_bounds__(kLrThreads, (lr_bwd_min_waves<E, W, GPV>())) void lr_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U,
    const E *__restrict__ dy, E *__restrict__ dx, float *__restrict__ dzp,
    float *__restrict__ dUp, int T, int D, int R, int TC, int nchunk, int ncb, int64_t N,
    float rho, int act) {
  const bool ACT = act != 0;  // wave-uniform
  using Gm = LrGeo<E, W, GPV>;
  using Sm = LrBwdSmem<E, W, GPV, RB>;
  constexpr bool BF = Gm::BF;
  constexpr int V = Gm::V, NU = Gm::NU, NG = Gm::NG, NP = Gm::NP, NS = Gm::NS;
  constexpr int KS = RB * (BF ? 1 : 4);
  constexpr int NDZ = BF ? (NS + 7) / 8 : NS;  // dz MFMAs per tile and rank block
  constexpr int NRB = Sm::nrb;                 // 16-row blocks of the wave's 4*NS slots
  constexpr int RP = 16 * RB;
  extern __shared__ __align__(16) unsigned char smem[];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, j = lane & 15;
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int cw = cb * Gm::CB + wave * Gm::CW;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int GW = (D / Gm::H) * W;
  const int64_t seq = (int64_t)b * T;

  E *dwt = reinterpret_cast<E *>(smem + wave * Sm::dwt_bytes);
  // rows 4*NS .. 16*NRB-1 pad the last MFMA block and stay zero
  for (int r = 4 * NS + (lane >> 4); r < 16 * NRB; r += 4) dwt[r * 16 + (lane & 15)] = (E)0;
  float *dzbuf = reinterpret_cast<float *>(smem + 4 * Sm::dwt_bytes);

  // resident operands: filter A fragments and dz A fragments (U columns)
  typename WFrag<BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV, KS>(U, GW, R, cw, D, lane, aw);
  typename DzFrag<BF>::T adz[NDZ][RB];
  {
    const int qa = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < NDZ; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rr = 16 * rb + r;
        if constexpr (BF) {
          bf16x8_t f;
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) {
            const int sg = 8 * s + e2;
            int col = -1;
            if (sg < NS) col = slot_col<E, W, GPV>(cw, qa, sg / NG, sg % NG, D);
            const uint16_t bits = (col >= 0 && rr < R) ? (uint16_t)U[(int64_t)rr * GW + col] : 0;
            f[e2] = __builtin_bit_cast(__bf16, bits);
          }
          adz[s][rb] = f;
        } else {
          const int col = slot_col<E, W, GPV>(cw, qa, s / NG, s % NG, D);
          adz[s][rb] = (col >= 0 && rr < R) ? (float)U[(int64_t)rr * GW + col] : 0.f;
        }
      }
  }

  f32x4 accU[NRB][RB];
#pragma unroll
  for (int a = 0; a < NRB; ++a)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) accU[a][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  float dxprev[NU][V];
  bool have_prev = false;
  int parity = 0;
  const int tiles = (t1 - t0 + 15) / 16;
  const int nsteps = tiles + (t1 < T ? 1 : 0);  // + a halo tile when tokens follow the chunk

  // Loads of one step, issued a step ahead and branch-free: a lane without a
  // token (past T) or a channel (past D) reads row 0 instead, and the value is
  // zeroed where it is used, so every lane runs the same instructions and the
  // DPP row shifts below always see defined data.
  typename WFrag<BF>::T zn[KS];
  uint4 dyn[NU], xn[NU], xp[NU];
  typedef typename std::conditional<BF, short, float>::type zt_t;
  zt_t ztn[4];  // z[t + 4qa + e][n]: the dU B operand (K = tokens)
  auto issue = [&](int st) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;
    const int tau = t + j;
    const bool in_seq = tau < T;
    load_zB<E, KS>(z, seq + tau, in_seq, R, q, zn);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = cw + (u * 4 + q) * V;
      const bool act_lane = in_seq && c < D;
      const int64_t off = act_lane ? (seq + tau) * D + c : 0;
      dyn[u] = ld16(dy + off);
      if (ACT || !halo) xn[u] = ld16(x + off);  // own row; taps come by DPP
    }
    if (!halo) {
      const int qa = lane >> 4, n = lane & 15;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int tk = BF ? t + 4 * qa + e2 : t + 4 * e2 + qa;
        const bool ok = tk < t1 && n < R;
        const E v = z[ok ? (seq + tk) * R + n : 0];
        if constexpr (BF) ztn[e2] = ok ? (short)v : (short)0;
        else ztn[e2] = ok ? (float)v : 0.f;
      }
    }
  };
  // x of the 16 tokens before the chunk (zero before the sequence start)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = cw + (u * 4 + q) * V;
    const int tb = t0 - 16 + j;
    const bool ok = tb >= 0 && c < D;
    xp[u] = sel4(ok, ld16(x + (ok ? (seq + tb) * D + c : 0)));
  }
  issue(0);

  for (int st = 0; st < nsteps; ++st) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;  // wave-uniform
    const int tau = t + j;
    const bool in_seq = tau < T;
    const bool in_chunk = !halo && tau < t1;

    typename WFrag<BF>::T bz[KS];
    uint4 dyr[NU], xc[NU];
    zt_t zt[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bz[ks] = zn[ks];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bool act_lane = in_seq && cw + (u * 4 + q) * V < D;
      dyr[u] = dyn[u];
      xc[u] = sel4(act_lane && (ACT || !halo), xn[u]);
    }
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) zt[e2] = ztn[e2];
    if (st + 1 < nsteps) issue(st + 1);

    f32x4 wacc[W][NP];
    gen_filters<E, W, GPV, KS>(aw, bz, wacc);

    const int tp = t - 16 + j;  // token of the previous tile held by this lane
    float dwv[NS];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = cw + (u * 4 + q) * V;
      const bool act_lane = in_seq && c < D;
      float dyv[V];
      unpack<E>(dyr[u], dyv);
#pragma unroll
      for (int i = 0; i < V; ++i) dyv[i] = act_lane ? dyv[i] : 0.f;
      // x tap k of this vector: token tau-k, by DPP from the lanes (and the
      // previous tile) that loaded it; zero before the sequence start
      auto xtap = [&](int k, float (&o)[V]) { unpack<E>(tap_vec(xc[u], xp[u], k), o); };
      float ds[V];
      if (ACT) {
        float sacc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float xk[V];
          xtap(k, xk);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const int m = u * GPV + i / Gm::H;
            sacc[i] = fmaf(wacc[k][m >> 2][m & 3], xk[i], sacc[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) ds[i] = dyv[i] * silu_grad_f(sacc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) ds[i] = dyv[i];
      }
      // input gradient: own tap 0; taps k >= 1 arrive from lane j+k of this
      // tile (row_shl) or go to lanes 16-k..15 of the previous tile (row_shr)
      float prev[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int m = u * GPV + i / Gm::H;
        float cur = fmaf(wacc[0][m >> 2][m & 3], ds[i], rho * dyv[i]);
        float pv = have_prev ? dxprev[u][i] : 0.f;
#pragma unroll
        for (int k = 1; k < W; ++k) {
          const float pk = wacc[k][m >> 2][m & 3] * ds[i];
          cur += row_shl(pk, k);
          pv += row_shr_16mk(pk, k);
        }
        prev[i] = pv;
        dxprev[u][i] = cur;  // becomes the previous tile at the next step
      }
      if (have_prev && tp < t1 && c < D) st16(dx + (seq + tp) * D + c, pack<E>(prev));
      // filter gradient slots of this vector (zero outside the chunk)
#pragma unroll
      for (int k = 0; k < W; ++k) {
        float xk[V];
        xtap(k, xk);
#pragma unroll
        for (int gi = 0; gi < GPV; ++gi) {
          float a = 0.f;
#pragma unroll
          for (int h = 0; h < Gm::H; ++h) a = fmaf(ds[gi * Gm::H + h], xk[gi * Gm::H + h], a);
          dwv[k * NG + u * GPV + gi] = in_chunk ? a : 0.f;
        }
      }
      xp[u] = xc[u];
    }
    have_prev = true;
    if (halo) break;

    // ---- dz^T (16 ranks x 16 tokens) over this wave's slots ----
    f32x4 dzacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) dzacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NDZ; ++s) {
      typename DzFrag<BF>::T bdw;
      if constexpr (BF) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          const int sg = 8 * s + e2;
          bdw[e2] = (__bf16)(sg < NS ? dwv[sg] : 0.f);
        }
      } else {
        bdw = dwv[s];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) dzacc[rb] = mma_dz<BF>(adz[s][rb], bdw, dzacc[rb]);
    }
    // sum the 4 waves' partials in a fixed order (LDS, double-buffered)
    float *zb = dzbuf + parity * (4 * RB * 64 * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      *reinterpret_cast<f32x4 *>(zb + ((wave * RB + rb) * 64 + lane) * 4) = dzacc[rb];
    __syncthreads();
    if (wave == 0 && tau < t1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 s4 = *reinterpret_cast<const f32x4 *>(zb + ((0 * RB + rb) * 64 + lane) * 4);
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) {
          const f32x4 o4 = *reinterpret_cast<const f32x4 *>(zb + ((w2 * RB + rb) * 64 + lane) * 4);
          s4 += o4;
        }
        // lane (q, j) holds ranks 16rb + 4q .. +3 of token tau
        *reinterpret_cast<f32x4 *>(dzp + ((int64_t)cb * N + seq + tau) * RP + 16 * rb + 4 * q) = s4;
      }
    }
    parity ^= 1;

    // ---- dU^T += dw^T z: transpose dw through LDS (row = slot*4 + quarter) ----
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      if constexpr (BF) {
        dwt[(sg * 4 + q) * 16 + j] = __builtin_bit_cast(uint16_t, (__bf16)dwv[sg]);
      } else {
        dwt[(sg * 4 + q) * 16 + j] = dwv[sg];
      }
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (BF) {
      // B operand: z[token 4qa+e2][16rb + n] (K = tokens)
      static_assert(RB == 1, "one rank block");
      const int qa = lane >> 4, n = lane & 15;
      s16x4 bzt[RB];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) bzt[0][e2] = zt[e2];
#pragma unroll
      for (int a = 0; a < NRB; ++a) {
        const uint2 v = *reinterpret_cast<const uint2 *>(dwt + (16 * a + n) * 16 + 4 * qa);
        s16x4 af;
        af[0] = (short)(v.x & 0xffff); af[1] = (short)(v.x >> 16);
        af[2] = (short)(v.y & 0xffff); af[3] = (short)(v.y >> 16);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          accU[a][rb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, bzt[rb], accU[a][rb], 0, 0, 0);
      }
    } else {
      static_assert(RB == 1, "one rank block");
      const int qa = lane >> 4, n = lane & 15;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        float bzt[RB];
        bzt[0] = zt[s4];
#pragma unroll
        for (int a = 0; a < NRB; ++a) {
          const float af = dwt[(16 * a + n) * 16 + 4 * s4 + qa];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            accU[a][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bzt[rb], accU[a][rb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // the last tile of the chunk when no halo followed (end of the sequence)
  if (t1 >= T && have_prev) {
    const int tp = t0 + 16 * (tiles - 1) + j;
    if (tp < t1) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = cw + (u * 4 + q) * V;
        if (c < D) st16(dx + (seq + tp) * D + c, pack<E>(dxprev[u]));
      }
    }
  }
  // dU partial of this chunk: lane (qo, n) holds rows 16a + 4qo + e
  // = (slot 4a + qo, quarter e) for rank 16rb + n
  {
    const int qo = lane >> 4, n = lane & 15;
    float *dst = dUp + (int64_t)(b * nchunk + chunk) * RP * GW;
#pragma unroll
    for (int a = 0; a < NRB; ++a) {
      const int sg = 4 * a + qo;
      if (sg >= NS) continue;  // padding rows of the last block
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = slot_col<E, W, GPV>(cw, e, sg / NG, sg % NG, D);
        if (col < 0) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) dst[(int64_t)(16 * rb + n) * GW + col] = accU[a][rb][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Deterministic reduction of the partials: dz = sum over channel blocks,
// dU = sum over chunks, each in ascending block order, then cast.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void lr_reduce_kernel(const float *__restrict__ dzp,
                                                        const float *__restrict__ dUp,
                                                        E *__restrict__ dz, E *__restrict__ dU,
                                                        int64_t N, int R, int RP, int ncb,
                                                        int64_t GW, int nparts) {
  const int64_t nz = N * R, nu = (int64_t)R * GW;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nz + nu;
       idx += (int64_t)gridDim.x * blockDim.x) {
    float acc = 0.f;
    if (idx < nz) {
      const int64_t n = idx / R;
      const int r = (int)(idx % R);
      for (int c = 0; c < ncb; ++c) acc += dzp[((int64_t)c * N + n) * RP + r];
      if constexpr (sizeof(E) == 2) {
        dz[idx] = __builtin_bit_cast(uint16_t, (__bf16)acc);
      } else {
        dz[idx] = acc;
      }
    } else {
      const int64_t o = idx - nz;
      const int64_t r = o / GW, col = o % GW;
      for (int c = 0; c < nparts; ++c) acc += dUp[((int64_t)c * RP + r) * GW + col];
      if constexpr (sizeof(E) == 2) {
        dU[o] = __builtin_bit_cast(uint16_t, (__bf16)acc);
      } else {
        dU[o] = acc;
      }
    }
  }
}

}  // namespace dsc
