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
// is z^T of 16 tokens (K = ranks) and whose A operand holds the U columns of
// the (group, tap k) slots the lanes need.  The output layout of a 16x16 MFMA
// gives lane (q, j) rows 4q..4q+3 of column j, so each lane receives exactly
// the tap-k filter of its own token and channels.  bf16 uses
// v_mfma_f32_16x16x16_bf16 (bf16 products, fp32 sums); fp32 uses
// v_mfma_f32_16x16x4_f32.
//
// Shifted rows.  The rows of other tokens (x at t-k for the taps, ds at t+k
// for dx) go through a 32-row LDS ring, written once per tile and read back
// with 16-byte LDS reads, so the shifts cost LDS bandwidth rather than
// vector-ALU issue.  The forward's ring spans the workgroup and is filled by
// row-major loads; its outputs leave through an LDS staging tile, so every
// device-memory access is a whole-row segment of the channel block.
//
// Backward per tile (one-tile lag for dx):
//   * ds = dy (or dy * SiLU'(s), s recomputed from the on-chip filters);
//   * dx[t] = rho dy[t] + sum_k w[t+k,k] ds[t+k] for the previous tile: the
//     filters w[t+k,.,k] come from MFMAs fed with z of token t+k, ds[t+k]
//     from the ds ring; a final step over the tokens after the chunk (zero
//     past the sequence end) completes the chunk's last tile;
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
  static constexpr int KS = BF ? 1 : 4;     // rank steps per filter MFMA (R <= 16)
  // LDS rings (per wave): 32 token rows of x (raw) and of ds (fp32), each row
  // padded by 16 bytes so that 16 consecutive rows spread over the banks
  static constexpr int XROW = CW * (int)sizeof(E) + 16;
  static constexpr int DROW = CW * 4 + 16;
};

// ---- small helpers -----------------------------------------------------------
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
// holds U[ranks of K-quarter qa][column of output row i]; row i = 4*qo + e of
// the output goes to lane quarter qo as slot m = 4p + e of tap k.
template <typename E, int W, int GPV>
__device__ __forceinline__ void load_wA(
    const E *__restrict__ U, int GW, int R, int cw, int D, int lane,
    typename WFrag<sizeof(E) == 2>::T (&a)[W][LrGeo<E, W, GPV>::NP][LrGeo<E, W, GPV>::KS]) {
  using Gm = LrGeo<E, W, GPV>;
  const int qa = lane >> 4, i = lane & 15, qo = i >> 2, e = i & 3;
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int p = 0; p < Gm::NP; ++p) {
      const int m = 4 * p + e;
      const int col = m < Gm::NG ? slot_col<E, W, GPV>(cw, qo, k, m, D) : -1;
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) {
        if constexpr (Gm::BF) {
          s16x4 f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = 4 * qa + e2;
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
// only ever multiply zeros, and ranks r >= R meet zero rows of U, so the
// fragment needs no masking.
template <typename E, int KS>
__device__ __forceinline__ void load_zB(const E *__restrict__ z, int64_t tok, bool valid, int R,
                                        int q, typename WFrag<sizeof(E) == 2>::T (&bz)[KS]) {
  constexpr bool BF = sizeof(E) == 2;
  const E *zr = z + (valid ? tok * R : 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (BF) {
      const int r0 = 4 * q;
      s16x4 f;
      if ((R & 3) == 0) {  // 8-byte aligned 4-rank groups, all in or all out
        // the raw bits are the fragment: no instruction touches the loaded
        // value before the MFMA, so the load stays in flight until then
        f = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(r0 < R ? zr + r0 : z));
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

// Tap-k filters of 16 tokens: acc[p][e] at lane (q, j) is the tap-k weight of
// slot m = 4p+e of the token whose z fragment is bz.
template <typename E, int W, int GPV>
__device__ __forceinline__ void gen_tap(
    const typename WFrag<sizeof(E) == 2>::T (&a)[LrGeo<E, W, GPV>::NP][LrGeo<E, W, GPV>::KS],
    const typename WFrag<sizeof(E) == 2>::T (&bz)[LrGeo<E, W, GPV>::KS],
    f32x4 (&acc)[LrGeo<E, W, GPV>::NP]) {
  using Gm = LrGeo<E, W, GPV>;
#pragma unroll
  for (int p = 0; p < Gm::NP; ++p) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Gm::KS; ++ks) c = mma_w<Gm::BF>(a[p][ks], bz[ks], c);
    acc[p] = c;
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// Device memory is touched only by whole-workgroup row segments: per tile the
// workgroup loads the 16 x CB slab of x (thread -> one 16-byte vector of a
// row, consecutive threads along the row) into a workgroup-wide fp32 ring of
// 32 token rows, the lanes compute in the token-per-lane layout reading the
// ring, and the 16 x CB slab of y goes back through an LDS staging tile with
// the same row-major thread mapping.  Loading and storing per lane (16 token
// rows of 64 bytes per instruction) ran at two thirds of this speed.
template <typename E, int W, int GPV> struct LrFwdGeo {
  using Gm = LrGeo<E, W, GPV>;
  static constexpr int XR = Gm::CB * 4 + 16;               // ring row pitch (fp32)
  static constexpr int SP = Gm::CB * (int)sizeof(E) + 16;  // staging row pitch
  static constexpr int VPR = Gm::CB / Gm::V;               // 16-byte vectors per row
  static constexpr int RPP = kLrThreads / VPR;             // rows per cooperative pass
  static constexpr int NPASS = 16 / RPP;                   // passes per 16-row slab
  static_assert(RPP * NPASS == 16, "a slab is a whole number of passes");
  static constexpr int bytes = 32 * XR + 16 * SP;
};

template <typename E, int W, int GPV, bool ACT>
__global__ __launch_bounds__(kLrThreads) void lr_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U, E *__restrict__ y,
    int T, int D, int R, int TC, int nchunk, int ncb, float rho) {
  using Gm = LrGeo<E, W, GPV>;
  using Fg = LrFwdGeo<E, W, GPV>;
  constexpr int V = Gm::V, NU = Gm::NU, NP = Gm::NP, KS = Gm::KS;
  constexpr int XR = Fg::XR, SP = Fg::SP, VPR = Fg::VPR, RPP = Fg::RPP, NPASS = Fg::NPASS;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *ring = smem, *stage = smem + 32 * XR;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, j = lane & 15;
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int cw = cb * Gm::CB + wave * Gm::CW;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int GW = (D / Gm::H) * W;
  const int64_t seq = (int64_t)b * T;
  // row-major role: vector vv of rows rr, rr + RPP, ...
  const int vv = tid % VPR, rr = tid / VPR;
  const int cc = cb * Gm::CB + vv * V;
  const bool cc_ok = cc < D;
  // ring row slot of token `tok` (any sign): tok & 31 is tok mod 32
  auto ring_put = [&](int tok, const uint4 &raw, bool ok) {
    float v[V];
    unpack<E>(sel4(ok, raw), v);
    f32x4 *dst = reinterpret_cast<f32x4 *>(ring + (tok & 31) * XR + vv * V * 4);
#pragma unroll
    for (int h = 0; h < V / 4; ++h) dst[h] = f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
  };
  // the V channels of lane vector u at token `tok`, as V/4 16-byte pieces
  auto xrow = [&](int tok, int u) {
    return reinterpret_cast<const f32x4 *>(ring + (tok & 31) * XR +
                                           (wave * Gm::CW + (u * 4 + q) * V) * 4);
  };

  typename WFrag<Gm::BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV>(U, GW, R, cw, D, lane, aw);

  // the 16 rows before the chunk (zero before the sequence)
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int tb = t0 - 16 + p * RPP + rr;
    const bool ok = tb >= 0 && cc_ok;
    ring_put(tb, ld16(x + (ok ? (seq + tb) * D + cc : 0)), ok);
  }
  // Loads of one tile go to one of PF prefetch slots, PF tiles ahead; they are
  // branch-free (a thread without a token or channel reads row 0, zeroed later).
  constexpr int PF = 4;
  typename WFrag<Gm::BF>::T zn[PF][KS];
  uint4 xn[PF][NPASS];
  auto issue = [&](int t, int sl) {  // sl: compile-time after unrolling
    load_zB<E, KS>(z, seq + t + j, t + j < t1, R, q, zn[sl]);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int tr = t + p * RPP + rr;
      xn[sl][p] = ld16(x + (tr < t1 && cc_ok ? (seq + tr) * D + cc : 0));
    }
  };
  // Per tile: fill the ring rows of the tile; barrier; taps, outputs to the
  // staging tile; barrier; row-major stores.  The next tile's fill overwrites
  // the rows of tile t-16, whose last reads precede the second barrier, and
  // its staging writes follow its own first barrier, after these stores read.
  auto tile = [&](int t, int sl) {
    const int tau = t + j;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int tr = t + p * RPP + rr;
      ring_put(tr, xn[sl][p], tr < t1 && cc_ok);
    }
    typename WFrag<Gm::BF>::T bz[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bz[ks] = zn[sl][ks];
    if (t + 16 * PF < t1) issue(t + 16 * PF, sl);  // workgroup-uniform
    f32x4 wacc[W][NP];
#pragma unroll
    for (int k = 0; k < W; ++k) gen_tap<E, W, GPV>(aw[k], bz, wacc[k]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float acc[V], x0[V];
#pragma unroll
      for (int h = 0; h < V / 4; ++h) {
        const f32x4 x4 = xrow(tau, u)[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) x0[4 * h + e] = x4[e];
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int m = u * GPV + i / Gm::H;
        acc[i] = wacc[0][m >> 2][m & 3] * x0[i];
      }
#pragma unroll
      for (int k = 1; k < W; ++k) {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
          const f32x4 x4 = xrow(tau - k, u)[h];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * h + e;
            const int m = u * GPV + i / Gm::H;
            acc[i] = fmaf(wacc[k][m >> 2][m & 3], x4[e], acc[i]);
          }
        }
      }
      float o[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float sv = acc[i];
        if constexpr (ACT) sv = silu_f(sv);
        o[i] = fmaf(rho, x0[i], sv);
      }
      *reinterpret_cast<uint4 *>(stage + j * SP + (wave * Gm::CW + (u * 4 + q) * V) * (int)sizeof(E)) =
          pack<E>(o);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int r = p * RPP + rr;
      const uint4 val = *reinterpret_cast<const uint4 *>(stage + r * SP + vv * 16);
      if (t + r < t1 && cc_ok) st16(y + (seq + t + r) * D + cc, val);
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (t0 + 16 * p < t1) issue(t0 + 16 * p, p);
  for (int t = t0; t < t1; t += 16 * PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (t + 16 * p < t1) tile(t + 16 * p, p);
  }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
template <typename E, int W, int GPV> struct LrBwdSmem {
  using Gm = LrGeo<E, W, GPV>;
  // per wave: dw^T, 4*NS slot rows x 16 tokens, padded with zero rows to
  // whole 16-row MFMA blocks
  static constexpr int nrb = (Gm::NS + 3) / 4;
  static constexpr int dwt_bytes = 16 * nrb * 16 * (int)sizeof(E);
  static constexpr int xring_bytes = 32 * Gm::XROW;
  static constexpr int dring_bytes = 32 * Gm::DROW;
  static constexpr int wave_bytes = dwt_bytes + xring_bytes + dring_bytes;
  // per workgroup: two buffers of the 4 waves' dz^T tiles (64 lanes x 4)
  static constexpr int dz_floats = 2 * 4 * 64 * 4;
  static constexpr int bytes = 4 * wave_bytes + dz_floats * 4;
};

// Two waves per SIMD (at most 256 VGPR+AGPR per lane) where the compiler fits
// that without spilling, one otherwise.  The set was read off the kernel
// resource-usage report of every instance.
template <typename E, int W, int GPV>
constexpr int lr_bwd_min_waves() {
  if constexpr (sizeof(E) == 2) {
    const bool two = (W == 1 && GPV != 2) || ((W == 2 || W == 3) && GPV == 4) ||
                     (W == 4 && (GPV == 1 || GPV == 8)) || (W == 5 && GPV == 8) ||
                     (W == 7 && (GPV == 1 || GPV == 2));
    return two ? 2 : 1;
  } else {
    const bool two = W <= 4 || (W == 5 && (GPV == 1 || GPV == 4)) ||
                     (W == 7 && (GPV == 1 || GPV == 2)) || (W == 8 && GPV == 1);
    return two ? 2 : 1;
  }
}

template <typename E, int W, int GPV>
__global__ __launch_bounds__(kLrThreads, (lr_bwd_min_waves<E, W, GPV>())) void lr_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U,
    const E *__restrict__ dy, E *__restrict__ dx, float *__restrict__ dzp,
    float *__restrict__ dUp, int T, int D, int R, int TC, int nchunk, int ncb, int64_t N,
    float rho, int act) {
  using Gm = LrGeo<E, W, GPV>;
  using Sm = LrBwdSmem<E, W, GPV>;
  constexpr bool BF = Gm::BF;
  constexpr int V = Gm::V, NU = Gm::NU, NG = Gm::NG, NP = Gm::NP, NS = Gm::NS, KS = Gm::KS;
  constexpr int NDZ = BF ? (NS + 7) / 8 : NS;  // dz MFMAs per tile
  constexpr int NRB = Sm::nrb;                 // 16-row blocks of the wave's 4*NS slots
  constexpr int RP = 16;
  constexpr int XROW = Gm::XROW, DROW = Gm::DROW;
  const bool ACT = act != 0;  // wave-uniform
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

  unsigned char *wbase = smem + wave * Sm::wave_bytes;
  E *dwt = reinterpret_cast<E *>(wbase);
  unsigned char *xring = wbase + Sm::dwt_bytes;
  unsigned char *dring = xring + Sm::xring_bytes;
  float *dzbuf = reinterpret_cast<float *>(smem + 4 * Sm::wave_bytes);
  auto xslot = [&](int tok, int u) {
    return reinterpret_cast<uint4 *>(xring + (tok & 31) * XROW + (u * 4 + q) * 16);
  };
  // ds ring: V fp32 of vector u at token tok, as V/4 16-byte pieces
  auto dslot = [&](int tok, int u) {
    return reinterpret_cast<f32x4 *>(dring + (tok & 31) * DROW + (u * 4 + q) * V * 4);
  };
  // rows 4*NS .. 16*NRB-1 pad the last dw^T MFMA block and stay zero
  for (int r = 4 * NS + (lane >> 4); r < 16 * NRB; r += 4) dwt[r * 16 + (lane & 15)] = (E)0;

  // resident operands: filter A fragments and dz A fragments (U columns)
  typename WFrag<BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV>(U, GW, R, cw, D, lane, aw);
  typename DzFrag<BF>::T adz[NDZ];
  {
    const int qa = lane >> 4, r = lane & 15;
#pragma unroll
    for (int s = 0; s < NDZ; ++s) {
      if constexpr (BF) {
        bf16x8_t f;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          const int sg = 8 * s + e2;
          int col = -1;
          if (sg < NS) col = slot_col<E, W, GPV>(cw, qa, sg / NG, sg % NG, D);
          const uint16_t bits = (col >= 0 && r < R) ? (uint16_t)U[(int64_t)r * GW + col] : 0;
          f[e2] = __builtin_bit_cast(__bf16, bits);
        }
        adz[s] = f;
      } else {
        const int col = slot_col<E, W, GPV>(cw, qa, s / NG, s % NG, D);
        adz[s] = (col >= 0 && r < R) ? (float)U[(int64_t)r * GW + col] : 0.f;
      }
    }
  }

  f32x4 accU[NRB];
#pragma unroll
  for (int a = 0; a < NRB; ++a) accU[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  // x rows of the 16 tokens before the chunk (zero before the sequence start)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = cw + (u * 4 + q) * V;
    const int tb = t0 - 16 + j;
    const bool ok = tb >= 0 && c < D;
    *xslot(tb, u) = sel4(ok, ld16(x + (ok ? (seq + tb) * D + c : 0)));
  }

  // Loads of one step, issued a step ahead and branch-free: a lane without a
  // token (past T) or a channel (past D) reads row 0 instead, and the value is
  // zeroed where it is used.
  typedef typename WFrag<BF>::T wfrag_t;
  typedef typename std::conditional<BF, short, float>::type zt_t;
  wfrag_t zn[KS];        // z of the step's own tokens (SiLU only)
  wfrag_t zsn[W][KS];    // z of tokens t-16+j+k: filters w[t'+k, ., k] for dx
  uint4 dyn[NU], xn[NU];
  zt_t ztn[4];           // z[t + 4qa + e][n]: the dU B operand (K = tokens);
                         // rows past the chunk meet zero dw rows, ranks n >= R
                         // give dU rows that are never read: no masking
  const int tiles = (t1 - t0 + 15) / 16;
  const int nsteps = tiles + 1;  // + the tokens after the chunk (dx of its last tile)
  // per-lane element offsets of the first tile's row, advanced by 16 rows a step
  int64_t row0[NU];
  bool chan_ok[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = cw + (u * 4 + q) * V;
    chan_ok[u] = c < D;
    row0[u] = (seq + t0 + j) * D + c;
  }
  auto issue = [&](int st) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;
    const int tau = t + j;
    const bool in_seq = tau < T;
    if (ACT) load_zB<E, KS>(z, seq + tau, in_seq, R, q, zn);
    if (st > 0) {
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int tk = t - 16 + j + k;
        load_zB<E, KS>(z, seq + tk, tk < T, R, q, zsn[k]);
      }
    }
    const int64_t step_off = (int64_t)(16 * st) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t off = in_seq && chan_ok[u] ? row0[u] + step_off : 0;
      dyn[u] = ld16(dy + off);
      if (ACT || !halo) xn[u] = ld16(x + off);
    }
    if (!halo) {
      const int qa = lane >> 4, n = lane & 15;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int tk = BF ? t + 4 * qa + e2 : t + 4 * e2 + qa;
        const bool ok = tk < t1 && n < R;
        if constexpr (BF) ztn[e2] = (short)z[ok ? (seq + tk) * R + n : 0];
        else ztn[e2] = z[ok ? (seq + tk) * R + n : 0];
      }
    }
  };
  issue(0);

  float dyp[NU][V];  // dy of the previous tile (residual term of its dx)
  int parity = 0;
  for (int st = 0; st < nsteps; ++st) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;  // wave-uniform
    const int tau = t + j;
    const bool in_seq = tau < T;

    wfrag_t bz[KS], bzs[W][KS];
    uint4 dyr[NU], xc[NU];
    zt_t zt[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bz[ks] = zn[ks];
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bzs[k][ks] = zsn[k][ks];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bool act_lane = in_seq && cw + (u * 4 + q) * V < D;
      dyr[u] = sel4(act_lane, dyn[u]);
      xc[u] = sel4(act_lane && (ACT || !halo), xn[u]);
    }
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) zt[e2] = ztn[e2];
    if (st + 1 < nsteps) issue(st + 1);

    // own x row into the ring (taps of later tokens)
    if (ACT || !halo) {
#pragma unroll
      for (int u = 0; u < NU; ++u) *xslot(tau, u) = xc[u];
    }
    __builtin_amdgcn_wave_barrier();
    // x tap k of vector u for this lane's token (zero before the sequence)
    auto xtap = [&](int u, int k, float (&o)[V]) {
      unpack<E>(k == 0 ? xc[u] : *xslot(tau - k, u), o);
    };

    // ds = dy (or dy * SiLU'(s)) of this tile's tokens, into the ds ring
    float ds[NU][V];
    if (ACT) {
      f32x4 wacc[W][NP];
#pragma unroll
      for (int k = 0; k < W; ++k) gen_tap<E, W, GPV>(aw[k], bz, wacc[k]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float sacc[V], dyv[V];
        unpack<E>(dyr[u], dyv);
#pragma unroll
        for (int i = 0; i < V; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float xk[V];
          xtap(u, k, xk);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const int m = u * GPV + i / Gm::H;
            sacc[i] = fmaf(wacc[k][m >> 2][m & 3], xk[i], sacc[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) ds[u][i] = dyv[i] * silu_grad_f(sacc[i]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) unpack<E>(dyr[u], ds[u]);  // ds = dy
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int h = 0; h < V / 4; ++h)
        dslot(tau, u)[h] = f32x4{ds[u][4 * h], ds[u][4 * h + 1], ds[u][4 * h + 2], ds[u][4 * h + 3]};
    __builtin_amdgcn_wave_barrier();

    // dx of the previous tile: dx[t'] = rho dy[t'] + sum_k w[t'+k,.,k] ds[t'+k]
    if (st > 0) {
      const int tp = t - 16 + j;
      float dxa[NU][V];
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) dxa[u][i] = rho * dyp[u][i];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        f32x4 wk[NP];
        gen_tap<E, W, GPV>(aw[k], bzs[k], wk);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const f32x4 *src = dslot(tp + k, u);
#pragma unroll
          for (int h = 0; h < V / 4; ++h) {
            const f32x4 d4 = src[h];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * h + e;
              const int m = u * GPV + i / Gm::H;
              dxa[u][i] = fmaf(wk[m >> 2][m & 3], d4[e], dxa[u][i]);
            }
          }
        }
      }
      if (tp < t1) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = cw + (u * 4 + q) * V;
          if (c < D) st16(dx + (seq + tp) * D + c, pack<E>(dxa[u]));
        }
      }
    }
    if (ACT) {
#pragma unroll
      for (int u = 0; u < NU; ++u) unpack<E>(dyr[u], dyp[u]);
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) dyp[u][i] = ds[u][i];
    }
    if (halo) break;

    // filter gradient slots of this tile.  A chunk ends inside a tile only at
    // the sequence end, where ds is already zero, so no lane needs masking.
    float dwv[NS];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int k = 0; k < W; ++k) {
        float xk[V];
        xtap(u, k, xk);
#pragma unroll
        for (int gi = 0; gi < GPV; ++gi) {
          float a = 0.f;
#pragma unroll
          for (int h = 0; h < Gm::H; ++h)
            a = fmaf(ds[u][gi * Gm::H + h], xk[gi * Gm::H + h], a);
          dwv[k * NG + u * GPV + gi] = a;
        }
      }
    }

    // dw as bf16 pairs (slots 2i, 2i+1), rounded once, used by both MFMAs
    constexpr int NPAIR = (NS + 1) / 2;
    uint32_t dwp[BF ? NPAIR : 1];
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < NPAIR; ++i)
        dwp[i] = pack_bf16x2(dwv[2 * i], 2 * i + 1 < NS ? dwv[2 * i + 1] : 0.f);
    }
    // ---- dz^T (16 ranks x 16 tokens) over this wave's slots ----
    f32x4 dzacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NDZ; ++s) {
      typename DzFrag<BF>::T bdw;
      if constexpr (BF) {
        uint4 v;
        v.x = 4 * s + 0 < NPAIR ? dwp[4 * s + 0] : 0u;
        v.y = 4 * s + 1 < NPAIR ? dwp[4 * s + 1] : 0u;
        v.z = 4 * s + 2 < NPAIR ? dwp[4 * s + 2] : 0u;
        v.w = 4 * s + 3 < NPAIR ? dwp[4 * s + 3] : 0u;
        bdw = __builtin_bit_cast(bf16x8_t, v);
      } else {
        bdw = dwv[s];
      }
      dzacc = mma_dz<BF>(adz[s], bdw, dzacc);
    }
    // sum the 4 waves' partials in a fixed order (LDS, double-buffered)
    float *zb = dzbuf + parity * (4 * 64 * 4);
    *reinterpret_cast<f32x4 *>(zb + (wave * 64 + lane) * 4) = dzacc;
    __syncthreads();
    if (wave == 0 && tau < t1) {
      f32x4 s4 = *reinterpret_cast<const f32x4 *>(zb + lane * 4);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) s4 += *reinterpret_cast<const f32x4 *>(zb + (w2 * 64 + lane) * 4);
      // lane (q, j) holds ranks 4q .. 4q+3 of token tau
      *reinterpret_cast<f32x4 *>(dzp + ((int64_t)cb * N + seq + tau) * RP + 4 * q) = s4;
    }
    parity ^= 1;

    // ---- dU^T += dw^T z: transpose dw through LDS (row = slot*4 + quarter) ----
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) {
      if constexpr (BF) {
        const uint32_t pr = dwp[sg >> 1];
        dwt[(sg * 4 + q) * 16 + j] = (uint16_t)((sg & 1) ? (pr >> 16) : (pr & 0xffffu));
      } else {
        dwt[(sg * 4 + q) * 16 + j] = dwv[sg];
      }
    }
    __builtin_amdgcn_wave_barrier();
    {
      const int qa = lane >> 4, n = lane & 15;
      if constexpr (BF) {
        s16x4 bzt;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) bzt[e2] = zt[e2];
#pragma unroll
        for (int a = 0; a < NRB; ++a) {
          const uint2 v = *reinterpret_cast<const uint2 *>(dwt + (16 * a + n) * 16 + 4 * qa);
          s16x4 af;
          af[0] = (short)(v.x & 0xffff); af[1] = (short)(v.x >> 16);
          af[2] = (short)(v.y & 0xffff); af[3] = (short)(v.y >> 16);
          accU[a] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, bzt, accU[a], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int a = 0; a < NRB; ++a) {
            const float af = dwt[(16 * a + n) * 16 + 4 * s4 + qa];
            accU[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, zt[s4], accU[a], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // dU partial of this chunk: lane (qo, n) holds rows 16a + 4qo + e
  // = (slot 4a + qo, quarter e) for rank n
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
        dst[(int64_t)n * GW + col] = accU[a][e];
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
