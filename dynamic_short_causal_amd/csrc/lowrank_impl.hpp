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
// chunk of tokens of one sequence; each wave owns CW = 4*V channels.  The
// workgroup walks its chunk in tiles of 16 tokens.  Device memory is touched
// by whole rows of the channel block (consecutive threads, consecutive
// 16-byte vectors) that go through LDS; inside a tile, lane (q, j)
// (q = lane / 16, j = lane % 16) computes token t+j and channel vector q of
// its wave's slice.
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
// for dx) come from 32-row fp32 LDS rings spanning the workgroup, filled once
// per tile by the row-major loads and read back with 16-byte LDS reads.
//
// Backward per tile (one-tile lag for dx):
//   * ds = dy (or dy * SiLU'(s), s recomputed from the on-chip filters);
//   * dw (on chip only) -> dz^T += U dw^T with 16x16x32 bf16 MFMAs (K = the
//     lane's slots), summed across the 4 waves in LDS and written as one fp32
//     partial per channel block;
//   * dU^T += dw^T z: dw is transposed through LDS, one 16-row block at a
//     time, so tokens become the K dimension; accumulated over the whole
//     chunk in registers and written once per chunk as an fp32 partial;
//   * dx[t] = rho dy[t] + sum_k w[t+k,k] ds[t+k] for the previous tile: the
//     filters w[t+k,.,k] come from MFMAs fed with z of token t+k (without
//     SiLU the residual is folded into the tap-0 filter: ds = dy), ds[t+k]
//     from the ds ring; a final step over the tokens after the chunk (zero
//     past the sequence end) completes the chunk's last tile.
// Where the x taps read for s stay in registers (see XR in the kernel), dw
// comes before dx so that, with SiLU, they serve dw at once.
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

// RB: blocks of 16 ranks (R <= 16 * RB)
template <typename E, int W, int GPV, int RB = 1> struct LrGeo {
  static constexpr bool BF = sizeof(E) == 2;
  static constexpr int V = Vw<E>::n;
  static constexpr int H = V / GPV;         // channels per filter group
  // one channel vector per lane: keeps the registers and LDS of the backward
  // small enough for three resident workgroups per CU
  static constexpr int NU = 1;
  static constexpr int NG = NU * GPV;       // (group, vector) instances per lane per tap
  static constexpr int NP = (NG + 3) / 4;   // filter MFMAs per tap (4 rows per lane each)
  static constexpr int NS = NG * W;         // filter slots per lane
  static constexpr int CW = 4 * NU * V;     // channels per wave
  static constexpr int CB = 4 * CW;         // channels per workgroup
  static constexpr int KS = BF ? RB : 4 * RB;  // filter MFMAs per output: 16 (bf16) or 4 ranks each
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

// Byte offset of channel vector vi (0..15; wave vi / 4, lane quarter vi % 4)
// in an fp32 ring row.  gfx950's LDS has 64 four-byte banks and serves a
// 16-byte read 16 lanes per pass; measured with a probe, a pass holds the
// lanes of one half-wave with equal parity of lane bits 2..4.  A ring read
// has lane (q, j) on row j + c and vector 4w + q, so a pass holds quarters q
// and q ^ 1 on complementary sets of 8 rows: placing those two vectors 256
// bytes (one turn of the banks) apart puts the pass on 16 distinct 4-bank
// windows, where the plain order put two lanes on one window.  bf16 rows only
// (16 vectors of 8 fp32, 512 bytes); fp32 rows (16 vectors of 16 bytes) keep
// the plain order, which would need twice the row to pair them.
template <typename E> __device__ __forceinline__ int ring_vec(int vi) {
  if constexpr (sizeof(E) == 2) return (2 * (vi >> 2) + ((vi & 3) >> 1)) * 32 + (vi & 1) * 256;
  else return vi * 16;
}
// Vector vv of a ring row from its V fp32 values.  For bf16 the two 16-byte
// halves go out in the opposite order on odd vectors, so that each of the
// two writes by 16 consecutive vectors covers 16 distinct 4-bank windows.
template <typename E>
__device__ __forceinline__ void ring_store(unsigned char *row, int vv, const float (&v)[Vw<E>::n]) {
  f32x4 *dst = reinterpret_cast<f32x4 *>(row + ring_vec<E>(vv));
  if constexpr (Vw<E>::n == 8) {
    const bool odd = vv & 1;
    const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    dst[odd ? 1 : 0] = odd ? b : a;
    dst[odd ? 0 : 1] = odd ? a : b;
  } else {
    dst[0] = f32x4{v[0], v[1], v[2], v[3]};
  }
}

// Filter slot sigma = k*NG + m of lane quarter qq; m = u*GPV + gi names vector
// u*4 + qq of the wave slice and group gi inside it.  Returns the column of
// the slot's filter in a (., G*W) matrix, or -1 when the channel lies beyond
// D.  With filters tied over more channels than a vector holds (H = hm * V,
// GPV = 1) the kernels tile by vector: the vector's own column is that of its
// group in a matrix of D/V groups (hm = 1: dU partials), U's column that of
// group c / H (hm = H / V).
template <typename E, int W, int GPV>
__device__ __forceinline__ int slot_col(int cw, int qq, int k, int m, int D, int hm = 1) {
  using Gm = LrGeo<E, W, GPV>;
  const int u = m / GPV, gi = m % GPV;
  const int c = cw + (u * 4 + qq) * Gm::V;
  if (c >= D) return -1;
  return ((c / Gm::H + gi) / hm) * W + k;
}

// A operands of the filter MFMAs: for tap k, part p, rank step ks, lane (qa, i)
// holds U[ranks of K-quarter qa][column of output row i]; row i = 4*qo + e of
// the output goes to lane quarter qo as slot m = 4p + e of tap k.
template <typename E, int W, int GPV, int RB>
__device__ __forceinline__ void load_wA(
    const E *__restrict__ U, int GW, int R, int cw, int D, int hm, int lane,
    typename WFrag<sizeof(E) == 2>::T (&a)[W][LrGeo<E, W, GPV, RB>::NP][LrGeo<E, W, GPV, RB>::KS]) {
  using Gm = LrGeo<E, W, GPV, RB>;
  const int qa = lane >> 4, i = lane & 15, qo = i >> 2, e = i & 3;
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int p = 0; p < Gm::NP; ++p) {
      const int m = 4 * p + e;
      const int col = m < Gm::NG ? slot_col<E, W, GPV>(cw, qo, k, m, D, hm) : -1;
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks) {
        if constexpr (Gm::BF) {
          s16x4 f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = 16 * ks + 4 * qa + e2;
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
      const int r0 = 16 * ks + 4 * q;
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
template <typename E, int W, int GPV, int RB>
__device__ __forceinline__ void gen_tap(
    const typename WFrag<sizeof(E) == 2>::T (&a)[LrGeo<E, W, GPV, RB>::NP][LrGeo<E, W, GPV, RB>::KS],
    const typename WFrag<sizeof(E) == 2>::T (&bz)[LrGeo<E, W, GPV, RB>::KS],
    f32x4 (&acc)[LrGeo<E, W, GPV, RB>::NP]) {
  using Gm = LrGeo<E, W, GPV, RB>;
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
// rows of 64 bytes per instruction) ran at two thirds of this speed.  x is
// loaded and y stored non-temporally (each is touched once per call).
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

// Packed rows (VL): taps k >= 1 of a token beyond its document position are
// zeroed right after the filters are formed, before any use.
template <typename E, int W, int GPV, bool ACT, bool VL, int RB>
__global__ __launch_bounds__(kLrThreads) void lr_fwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U,
    const int32_t *__restrict__ pos, E *__restrict__ y, int T, int D, int R, int TC,
    int nchunk, int ncb, float rho, int hm) {
  using Gm = LrGeo<E, W, GPV, RB>;
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
  const int GW = (D / Gm::H / hm) * W;  // U's row: D / H groups of W taps
  const int64_t seq = (int64_t)b * T;
  // row-major role: vector vv of rows rr, rr + RPP, ...
  const int vv = tid % VPR, rr = tid / VPR;
  const int cc = cb * Gm::CB + vv * V;
  const bool cc_ok = cc < D;
  // ring row slot of token `tok` (any sign): tok & 31 is tok mod 32
  static_assert(Gm::CB == 16 * V && NU == 1, "16 channel vectors per ring row");
  auto ring_put = [&](int tok, const uint4 &raw, bool ok) {
    float v[V];
    unpack<E>(sel4(ok, raw), v);
    ring_store<E>(ring + (tok & 31) * XR, vv, v);
  };
  // the V channels of lane vector u at token `tok`, as V/4 16-byte pieces
  auto xrow = [&](int tok, int u) {
    return reinterpret_cast<const f32x4 *>(ring + (tok & 31) * XR + ring_vec<E>(wave * 4 + u * 4 + q));
  };

  typename WFrag<Gm::BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV, RB>(U, GW, R, cw, D, hm, lane, aw);

  // the 16 rows before the chunk (zero before the sequence)
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int tb = t0 - 16 + p * RPP + rr;
    const bool ok = tb >= 0 && cc_ok;
    ring_put(tb, ld16nt(x + (ok ? (seq + tb) * D + cc : 0)), ok);
  }
  // Loads of one tile go to one of PF prefetch slots, PF tiles ahead; they are
  // branch-free (a thread without a token or channel reads row 0, zeroed later).
  constexpr int PF = 4;
  typename WFrag<Gm::BF>::T zn[PF][KS];
  uint4 xn[PF][NPASS];
  int pn[PF];  // document position of the lane's token (VL)
  auto issue = [&](int t, int sl) {  // sl: compile-time after unrolling
    load_zB<E, KS>(z, seq + t + j, t + j < t1, R, q, zn[sl]);
    if constexpr (VL) pn[sl] = pos[seq + min(t + j, t1 - 1)];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int tr = t + p * RPP + rr;
      xn[sl][p] = ld16nt(x + (tr < t1 && cc_ok ? (seq + tr) * D + cc : 0));
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
    const int pj = VL ? pn[sl] : 0;
    if (t + 16 * PF < t1) issue(t + 16 * PF, sl);  // workgroup-uniform
    f32x4 wacc[W][NP];
#pragma unroll
    for (int k = 0; k < W; ++k) gen_tap<E, W, GPV, RB>(aw[k], bz, wacc[k]);
    if constexpr (VL) {
#pragma unroll
      for (int k = 1; k < W; ++k)
        if (k > pj)
#pragma unroll
          for (int p = 0; p < NP; ++p) wacc[k][p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
      if (t + r < t1 && cc_ok) st16nt(y + (seq + t + r) * D + cc, val);
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
// Device memory is read and written through buffer resources covering one
// 16-token slab each: rows past the sequence (or channels past D, given an
// offset above the resource size) read as zero and are not written, so no
// load or store needs a mask or 64-bit address arithmetic.
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc mk_rsrc(const void *p, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;
// cache-policy operand of the buffer accesses: non-temporal (x, dy, dx are
// each touched once per call)
constexpr int kNT = 2;

template <typename E, int W, int GPV, int RB> struct LrBwdGeo {
  using Gm = LrGeo<E, W, GPV, RB>;
  static constexpr int RS = (int)sizeof(E);
  static constexpr int XP = Gm::CB * 4 + 16;   // x ring row pitch (fp32)
  static constexpr int DP = Gm::CB * 4 + 16;   // ds ring row pitch (fp32)
  static constexpr int SP = Gm::CB * RS + 16;  // dx staging row pitch
  // z ring row: 16 * RB ranks + 8 bytes, so 16 lanes reading 16 rows hit distinct banks
  static constexpr int ZP = 16 * RB * RS + 8;
  static constexpr int VPR = Gm::CB / Gm::V;
  static constexpr int RPP = kLrThreads / VPR;
  static constexpr int NPASS = 16 / RPP;
  static_assert(RPP * NPASS == 16, "a slab is a whole number of passes");
  static constexpr int nrb = (Gm::NS + 3) / 4;
  static constexpr int DWP = 20;  // dw^T block row: 16 tokens + 4 (bank spread)
  static constexpr int dwt_wave = 2 * 16 * DWP * RS;
  static constexpr int o_x = 0;
  static constexpr int o_ds = o_x + 32 * XP;
  static constexpr int o_dx = o_ds + 32 * DP;
  static constexpr int o_z = o_dx + 16 * SP;
  static constexpr int o_dz = o_z + 32 * ZP;
  static constexpr int o_dwt = o_dz + 4 * 64 * 16;
  static constexpr int o_pos = o_dwt + 4 * dwt_wave;  // 32 document positions (VL)
  static constexpr int bytes = o_pos + 32 * 4;
};

template <typename E, int W, int GPV, int RB>
__device__ __forceinline__ void gen_tap_init(
    const typename WFrag<sizeof(E) == 2>::T (&a)[LrGeo<E, W, GPV, RB>::NP][LrGeo<E, W, GPV, RB>::KS],
    const typename WFrag<sizeof(E) == 2>::T (&bz)[LrGeo<E, W, GPV, RB>::KS],
    f32x4 (&acc)[LrGeo<E, W, GPV, RB>::NP], float init) {
  using Gm = LrGeo<E, W, GPV, RB>;
#pragma unroll
  for (int p = 0; p < Gm::NP; ++p) {
    f32x4 c = {init, init, init, init};
#pragma unroll
    for (int ks = 0; ks < Gm::KS; ++ks) c = mma_w<Gm::BF>(a[p][ks], bz[ks], c);
    acc[p] = c;
  }
}

// Three waves per SIMD where the compiler fits that without spilling, fewer
// otherwise; the set was read off the kernel resource-usage report.
template <typename E, int W, int GPV, bool VL, int RB>
constexpr int lr_bwd_min_waves() {
  // more than 16 ranks: filter fragments of every rank block stay resident
  if constexpr (RB > 1) return 1;
  // packed rows' position ring takes the per-channel W = 4 case over
  if constexpr (VL && sizeof(E) == 2 && GPV == 8 && W == 4) return 2;
  if constexpr (sizeof(E) == 2)
    return (GPV == 8 && W == 8) || (VL && GPV == 8 && W == 7) ? 1
           : (GPV == 8 && W >= 5) || (GPV == 4 && W >= 7) ? 2
                                                          : 3;
  else return (GPV == 4 && W >= 7) || (GPV == 2 && W == 8) ? 2 : 3;
}

// Packed rows (VL): a 32-entry ring of document positions beside the z ring;
// a tap k >= 1 of token t is zeroed where k > pos[t], in the filters of dx and
// of the SiLU recomputation and in dw (hence in dz and dU).
//
// More than 16 ranks (RB > 1): the filters use every rank, and dz and dU are
// formed for one block of 16 ranks, rb0, per launch; the launcher runs one
// pass per block, the first of which also writes dx (do_dx).
template <typename E, int W, int GPV, bool VL, int RB>
__global__ __launch_bounds__(kLrThreads, (lr_bwd_min_waves<E, W, GPV, VL, RB>())) void lr_bwd_kernel(
    const E *__restrict__ x, const E *__restrict__ z, const E *__restrict__ U,
    const E *__restrict__ dy, const int32_t *__restrict__ pos, E *__restrict__ dx,
    float *__restrict__ dzp, float *__restrict__ dUp, int T, int D, int R, int TC, int nchunk,
    int ncb, int64_t N, float rho, int act, int rb0, int do_dx, int hm) {
  using Gm = LrGeo<E, W, GPV, RB>;
  using Bg = LrBwdGeo<E, W, GPV, RB>;
  constexpr bool BF = Gm::BF;
  constexpr int V = Gm::V, NU = Gm::NU, NG = Gm::NG, NP = Gm::NP, NS = Gm::NS, KS = Gm::KS;
  constexpr int NDZ = BF ? (NS + 7) / 8 : NS;
  constexpr int NRB = Bg::nrb;
  constexpr int RP = 16 * RB, RS = Bg::RS;
  constexpr int XP = Bg::XP, DP = Bg::DP, SP = Bg::SP, ZP = Bg::ZP, VPR = Bg::VPR, RPP = Bg::RPP,
                NPASS = Bg::NPASS;
  constexpr int PF = 1;  // loads one step ahead: a step outlasts the load latency
  // With SiLU the x taps read for the recomputation of s stay in registers for
  // dw, where the instance keeps its occupancy without spilling (W <= 4, fewer
  // than 8 groups per vector); the others read them from the ring again.
  constexpr bool XR = W <= 4 && GPV < 8;
  const bool ACT = act != 0;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *xring = smem + Bg::o_x, *dring = smem + Bg::o_ds, *dxstage = smem + Bg::o_dx,
                *zring = smem + Bg::o_z;
  float *dzbuf = reinterpret_cast<float *>(smem + Bg::o_dz);
  int *pring = reinterpret_cast<int *>(smem + Bg::o_pos);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, j = lane & 15;
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int cw = cb * Gm::CB + wave * Gm::CW;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int GWp = (D / Gm::H) * W;  // a dU partial row: one group per vector or finer
  const int GW = GWp / hm;          // U's row: D / H groups of W taps
  const int64_t seq = (int64_t)b * T;
  E *dwt = reinterpret_cast<E *>(smem + Bg::o_dwt + wave * Bg::dwt_wave);

  // row-major role: vector vv of rows rr + p*RPP; byte offsets inside a 16-row slab
  const int vv = tid % VPR, rr = tid / VPR;
  const int cc = cb * Gm::CB + vv * V;
  const uint32_t cbase = cc < D ? (uint32_t)cc * RS : kOOB;
  uint32_t voff[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) voff[p] = cbase + (uint32_t)((p * RPP + rr) * D * RS);
  const int lcol = wave * Gm::CW;
  static_assert(Gm::CB == 16 * V && NU == 1, "16 channel vectors per ring row");
  auto xslot = [&](int tok, int u) {
    return reinterpret_cast<const f32x4 *>(xring + (tok & 31) * XP + ring_vec<E>(wave * 4 + u * 4 + q));
  };
  auto dslot = [&](int tok, int u) {
    return reinterpret_cast<f32x4 *>(dring + (tok & 31) * DP + ring_vec<E>(wave * 4 + u * 4 + q));
  };
  auto zrow = [&](int tok) { return reinterpret_cast<const E *>(zring + (tok & 31) * ZP); };
  auto zfrag = [&](int tok, typename WFrag<BF>::T (&f)[KS]) {
    const E *zr = zrow(tok);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (BF) f[ks] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(zr + 16 * ks + 4 * q));
      else f[ks] = zr[ks * 4 + q];
    }
  };
  // 16-token slab resources: rows t .. t+15 of a [B*T, D] tensor, bounded by `lim`
  auto slab = [&](const E *base, int t, int lim) {
    return mk_rsrc(base + (seq + t) * (int64_t)D, (int64_t)(min(lim, t + 16) - t) * D * RS);
  };
  // the 16 x R values of a z slab, RB per thread: value zi = tid + 256 * i
  uint32_t zoff[RB];
  int zslot[RB];  // element offset of the value in a z ring row block, or -1
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int zi = tid + kLrThreads * i;
    const bool on = zi < 16 * R;
    zoff[i] = on ? (uint32_t)zi * RS : kOOB;
    const int tok = zi / (R > 0 ? R : 1), rank = zi - tok * (R > 0 ? R : 1);
    zslot[i] = on ? tok * (ZP / RS) + rank : -1;
  }
  auto zslab = [&](int t, int lim) {
    return mk_rsrc(z + (seq + t) * (int64_t)R, (int64_t)(min(lim, t + 16) - t) * R * RS);
  };
  // ring row of token t0 + 16 m + r is (t0 + 16 m + r) & 31: the 16 rows of a
  // slab starting at a multiple of 16 are contiguous in the ring
  auto zput = [&](int t, int i, E v) {
    if (zslot[i] >= 0) reinterpret_cast<E *>(zring + (t & 31) * ZP)[zslot[i]] = v;
  };

  for (int i = tid; i < 32 * ZP / 4; i += kLrThreads) reinterpret_cast<uint32_t *>(zring)[i] = 0u;

  typename WFrag<BF>::T aw[W][NP][KS];
  load_wA<E, W, GPV, RB>(U, GW, R, cw, D, hm, lane, aw);
  typename DzFrag<BF>::T adz[NDZ];
  {
    const int qa = lane >> 4, r = 16 * rb0 + (lane & 15);
#pragma unroll
    for (int s = 0; s < NDZ; ++s) {
      if constexpr (BF) {
        bf16x8_t f;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) {
          const int sg = 8 * s + e2;
          int col = -1;
          if (sg < NS) col = slot_col<E, W, GPV>(cw, qa, sg / NG, sg % NG, D, hm);
          const uint16_t bits = (col >= 0 && r < R) ? (uint16_t)U[(int64_t)r * GW + col] : 0;
          f[e2] = __builtin_bit_cast(__bf16, bits);
        }
        adz[s] = f;
      } else {
        const int col = slot_col<E, W, GPV>(cw, qa, s / NG, s % NG, D, hm);
        adz[s] = (col >= 0 && r < R) ? (float)U[(int64_t)r * GW + col] : 0.f;
      }
    }
  }
  f32x4 accU[NRB];
#pragma unroll
  for (int a = 0; a < NRB; ++a) accU[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int tiles = (t1 - t0 + 15) / 16;
  __syncthreads();  // z ring zeroed
  // prologue: x and z of the 16 tokens before the chunk (none before the sequence)
  {
    const int tb = t0 - 16;
    const brsrc rx = slab(x, tb, tb < 0 ? tb : T);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const uint4 raw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff[p], 0, 0));
      float v[V];
      unpack<E>(raw, v);
      ring_store<E>(xring + ((tb + p * RPP + rr) & 31) * XP, vv, v);
    }
    const brsrc rz = zslab(tb, tb < 0 ? tb : T);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      E v;
      if constexpr (BF) v = (E)__builtin_amdgcn_raw_buffer_load_b16(rz, zoff[i], 0, 0);
      else v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[i], 0, 0));
      zput(tb, i, v);
    }
  }

  uint4 xn[PF][NPASS], dyn[PF][NPASS];
  E zn[PF][RB];
  int pn[PF];
  auto issue = [&](int st, int sl) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;
    if constexpr (VL) {
      const brsrc rp = mk_rsrc(pos + seq + t, (int64_t)(min(T, t + 16) - t) * 4);
      pn[sl] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, tid < 16 ? (uint32_t)tid * 4 : kOOB, 0, 0);
    }
    const brsrc rdy = slab(dy, t, T);
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
      dyn[sl][p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rdy, voff[p], 0, kNT));
    if (ACT || !halo) {
      const brsrc rx = slab(x, t, T);
#pragma unroll
      for (int p = 0; p < NPASS; ++p)
        xn[sl][p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff[p], 0, kNT));
    }
    const brsrc rz = zslab(t, T);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if constexpr (BF) zn[sl][i] = (E)__builtin_amdgcn_raw_buffer_load_b16(rz, zoff[i], 0, 0);
      else zn[sl][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[i], 0, 0));
    }
  };
  auto fill = [&](int st, int sl) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int row = (t + p * RPP + rr) & 31;
      float v[V];
      unpack<E>(dyn[sl][p], v);
      ring_store<E>(dring + row * DP, vv, v);
      if (ACT || !halo) {
        float w[V];
        unpack<E>(xn[sl][p], w);
        ring_store<E>(xring + row * XP, vv, w);
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) zput(t, i, zn[sl][i]);
    if (VL && tid < 16) pring[(t + tid) & 31] = pn[sl];
  };

  float dyp[NU][V];  // (SiLU only) dy of the previous tile, for the residual term of its dx
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int i = 0; i < V; ++i) dyp[u][i] = 0.f;
  const float rho_act = ACT ? rho : 0.f;   // residual through dy (SiLU)
  const float rho_tap = ACT ? 0.f : rho;   // residual folded into the tap-0 filter (ds = dy)
  // The device stores of step st (dx of tile st-1 from the staging rows; the dz
  // partial of tile st, summed over the 4 waves in wave order) are issued at
  // the start of step st + 1, after its fill and before its prefetch.  Stores
  // count in the same counter as loads, so the fill's wait for its prefetched
  // rows then never waits for stores issued after those loads.
  auto flush = [&](int st) {
    const int t = t0 + 16 * st;
    if (st > 0 && do_dx) {
      const brsrc rdx = slab(dx, t - 16, t1);
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const uint4 val = *reinterpret_cast<const uint4 *>(dxstage + (p * RPP + rr) * SP + vv * 16);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, val), rdx, voff[p], 0, kNT);
      }
    }
    if (st < tiles && wave == 0 && t + j < t1) {
      f32x4 s4 = *reinterpret_cast<const f32x4 *>(dzbuf + lane * 4);
#pragma unroll
      for (int w2 = 1; w2 < 4; ++w2) s4 += *reinterpret_cast<const f32x4 *>(dzbuf + (w2 * 64 + lane) * 4);
      *reinterpret_cast<f32x4 *>(dzp + ((int64_t)cb * N + seq + t + j) * RP + 16 * rb0 + 4 * q) = s4;
    }
  };
  // halo_c: std::true_type for the last step (tokens after the chunk, dx
  // only).  Resolving it at compile time keeps every dU accumulation of the
  // main steps unconditional, so the accumulators stay in place across them.
  static_assert(PF == 1, "one step of loads in flight");
  auto step = [&](int st, auto halo_c) {
    constexpr bool halo = decltype(halo_c)::value;
    constexpr int sl = 0;
    const int t = t0 + 16 * st;
    const int tau = t + j;
    fill(st, sl);
    if (st > 0) flush(st - 1);
    if (!halo) issue(st + 1, sl);
    __syncthreads();  // (1) rings and slabs of this step written; staging and dz tiles of the last read
    float dxa[NU][V];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < V; ++i) dxa[u][i] = rho_act * dyp[u][i];
    // own ds (= dy, or dy * SiLU'(s))
    float ds[NU][V];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int h = 0; h < V / 4; ++h) {
        const f32x4 d4 = dslot(tau, u)[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[u][4 * h + e] = d4[e];
      }
    // x taps of the lane's token (x[tau - k]), for dw
    float xr[W][NU][V];
    if (ACT) {
      typename WFrag<BF>::T bz[KS];
      zfrag(tau, bz);
      f32x4 wacc[W][NP];
#pragma unroll
      for (int k = 0; k < W; ++k) gen_tap<E, W, GPV, RB>(aw[k], bz, wacc[k]);
      if constexpr (VL) {
        const int pj = pring[tau & 31];
#pragma unroll
        for (int k = 1; k < W; ++k)
          if (k > pj)
#pragma unroll
            for (int p = 0; p < NP; ++p) wacc[k][p] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float sacc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
          for (int h = 0; h < V / 4; ++h) {
            const f32x4 x4 = xslot(tau - k, u)[h];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * h + e, m = u * GPV + i / Gm::H;
              if constexpr (XR) xr[k][u][i] = x4[e];
              sacc[i] = fmaf(wacc[k][m >> 2][m & 3], x4[e], sacc[i]);
            }
          }
#pragma unroll
        for (int i = 0; i < V; ++i) {
          dyp[u][i] = ds[u][i];
          ds[u][i] = ds[u][i] * silu_grad_f(sacc[i]);
        }
#pragma unroll
        for (int h = 0; h < V / 4; ++h)
          dslot(tau, u)[h] = f32x4{ds[u][4 * h], ds[u][4 * h + 1], ds[u][4 * h + 2], ds[u][4 * h + 3]};
      }
    }
    // dx of the previous tile: dx[t'] = rho dy[t'] + sum_k w[t'+k,.,k] ds[t'+k]
    // (the wave barrier makes this wave's ds rows of the step visible)
    auto dx_part = [&]() {
      __builtin_amdgcn_wave_barrier();
      if (st > 0 && do_dx) {
        const int tp = t - 16 + j;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          typename WFrag<BF>::T bzs[KS];
          zfrag(tp + k, bzs);
          f32x4 wk[NP];
          gen_tap_init<E, W, GPV, RB>(aw[k], bzs, wk, k == 0 ? rho_tap : 0.f);
          if (VL && k > 0 && k > pring[(tp + k) & 31])
#pragma unroll
            for (int p = 0; p < NP; ++p) wk[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const f32x4 *src = dslot(tp + k, u);
#pragma unroll
            for (int h = 0; h < V / 4; ++h) {
              const f32x4 d4 = src[h];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 4 * h + e, m = u * GPV + i / Gm::H;
                dxa[u][i] = fmaf(wk[m >> 2][m & 3], d4[e], dxa[u][i]);
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *reinterpret_cast<uint4 *>(dxstage + j * SP + (lcol + (u * 4 + q) * V) * RS) = pack<E>(dxa[u]);
      }
    };
    if constexpr (!XR) dx_part();
    if constexpr (!halo) {
      // filter-gradient slots; a chunk ends inside a tile only at the sequence
      // end, where ds is zero, so no lane needs masking
      float dwv[NS];
      const int pown = VL ? pring[tau & 31] : W;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float xk[V];
          if (XR && ACT) {
#pragma unroll
            for (int i = 0; i < V; ++i) xk[i] = xr[k][u][i];
          } else {
#pragma unroll
            for (int h = 0; h < V / 4; ++h) {
              const f32x4 x4 = xslot(tau - k, u)[h];
#pragma unroll
              for (int e = 0; e < 4; ++e) xk[4 * h + e] = x4[e];
            }
          }
#pragma unroll
          for (int gi = 0; gi < GPV; ++gi) {
            float a = 0.f;
#pragma unroll
            for (int h = 0; h < Gm::H; ++h) a = fmaf(ds[u][gi * Gm::H + h], xk[gi * Gm::H + h], a);
            dwv[k * NG + u * GPV + gi] = (VL && k > 0 && k > pown) ? 0.f : a;
          }
        }
      constexpr int NPAIR = (NS + 1) / 2;
      uint32_t dwp[BF ? NPAIR : 1];
      if constexpr (BF) {
#pragma unroll
        for (int i = 0; i < NPAIR; ++i)
          dwp[i] = pack_bf16x2(dwv[2 * i], 2 * i + 1 < NS ? dwv[2 * i + 1] : 0.f);
      }
      f32x4 dzacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < NDZ; ++s2) {
        typename DzFrag<BF>::T bdw;
        if constexpr (BF) {
          uint4 v;
          v.x = 4 * s2 + 0 < NPAIR ? dwp[4 * s2 + 0] : 0u;
          v.y = 4 * s2 + 1 < NPAIR ? dwp[4 * s2 + 1] : 0u;
          v.z = 4 * s2 + 2 < NPAIR ? dwp[4 * s2 + 2] : 0u;
          v.w = 4 * s2 + 3 < NPAIR ? dwp[4 * s2 + 3] : 0u;
          bdw = __builtin_bit_cast(bf16x8_t, v);
        } else {
          bdw = dwv[s2];
        }
        dzacc = mma_dz<BF>(adz[s2], bdw, dzacc);
      }
      *reinterpret_cast<f32x4 *>(dzbuf + (wave * 64 + lane) * 4) = dzacc;
      // dU^T += dw^T z, one 16-row block (slots 4a..4a+3 of every quarter) at a time
      const int qa = lane >> 4, n = lane & 15;
      // z of rank 16 * rb0 + n (this pass's block)
      typename WFrag<BF>::T bzt[BF ? 1 : 4];
      if constexpr (BF) {
        s16x4 f;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) f[e2] = (short)zrow(t + 4 * qa + e2)[16 * rb0 + n];
        bzt[0] = f;
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) bzt[s4] = zrow(t + 4 * s4 + qa)[16 * rb0 + n];
      }
#pragma unroll
      for (int a = 0; a < NRB; ++a) {
        E *blk = dwt + (a & 1) * 256;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sg = 4 * a + e;
          E v = (E)0;
          if (sg < NS) {
            if constexpr (BF) {
              const uint32_t pr = dwp[sg >> 1];
              v = (uint16_t)((sg & 1) ? (pr >> 16) : (pr & 0xffffu));
            } else {
              v = dwv[sg];
            }
          }
          blk[(e * 4 + q) * 16 + j] = v;
        }
        __builtin_amdgcn_wave_barrier();
        if constexpr (BF) {
          const uint2 v = *reinterpret_cast<const uint2 *>(blk + n * 16 + 4 * qa);
          accU[a] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v), bzt[0], accU[a], 0, 0, 0);
        } else {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            accU[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(blk[n * 16 + 4 * s4 + qa], bzt[s4], accU[a], 0, 0, 0);
        }
      }
    }
    if constexpr (XR) dx_part();
    __syncthreads();  // (2) dx staging and dz partials complete; ring reads done
  };
  issue(0, 0);
  for (int st = 0; st < tiles; ++st) step(st, std::false_type{});
  step(tiles, std::true_type{});
  flush(tiles);
  {
    const int qo = lane >> 4, n = lane & 15;
    float *dst = dUp + (int64_t)(b * nchunk + chunk) * RP * GWp;
#pragma unroll
    for (int a = 0; a < NRB; ++a) {
      const int sg = 4 * a + qo;
      if (sg >= NS) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = slot_col<E, W, GPV>(cw, e, sg / NG, sg % NG, D);
        if (col < 0) continue;
        dst[(int64_t)(16 * rb0 + n) * GWp + col] = accU[a][e];
      }
    }
  }
}

// partial sums in a fixed order, loads issued 8 at a time
template <typename E>
__global__ __launch_bounds__(256) void lr_reduce_kernel(const float *__restrict__ dzp,
                                                         const float *__restrict__ dUp,
                                                         E *__restrict__ dz, E *__restrict__ dU,
                                                         int64_t N, int R, int RP, int ncb,
                                                         int64_t GW, int nparts, int W, int hm) {
  // dU is R x GW (GW = G*W); a partial row holds hm times as many groups when
  // filters are tied over hm vectors (one group per vector in the kernels),
  // and dU sums the hm adjacent groups of its own after the parts
  const int64_t GWp = GW * hm;
  const int64_t nz = N * R, nu = (int64_t)R * GW;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nz + nu;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const float *src;
    int64_t stride;
    int cnt;
    if (idx < nz) {
      const int64_t n = idx / R;
      const int r = (int)(idx - n * R);
      src = dzp + n * RP + r; stride = N * RP; cnt = ncb;
    } else {
      const int64_t o = idx - nz;
      const int64_t r = o / GW, col = o - r * GW;
      const int64_t g = col / W, k = col - g * W;
      src = dUp + r * GWp + g * hm * W + k; stride = (int64_t)RP * GWp; cnt = nparts;
    }
    float acc = 0.f;
    if (idx >= nz && hm > 1) {
      for (int c = 0; c < cnt; ++c)
        for (int i = 0; i < hm; ++i) acc += src[c * stride + i * W];
    } else {
      int c = 0;
      for (; c + 8 <= cnt; c += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = src[(c + i) * stride];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
      }
      for (; c < cnt; ++c) acc += src[c * stride];
    }
    if constexpr (sizeof(E) == 2) {
      if (idx < nz) dz[idx] = __builtin_bit_cast(uint16_t, (__bf16)acc);
      else dU[idx - nz] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    } else {
      if (idx < nz) dz[idx] = acc;
      else dU[idx - nz] = acc;
    }
  }
}

// The same sums, four consecutive outputs per thread with 16-byte loads of
// the partials (R and G*W multiples of 4, so that four consecutive outputs
// share a token row of dz or a rank row of dU; filters tied over at most one
// vector).  Same order of addition per output, so the same bits.
template <typename E>
__global__ __launch_bounds__(256) void lr_reduce4_kernel(const float *__restrict__ dzp,
                                                          const float *__restrict__ dUp,
                                                          E *__restrict__ dz, E *__restrict__ dU,
                                                          int64_t N, int R, int RP, int ncb,
                                                          int64_t GW, int nparts) {
  const int64_t nz = N * R / 4, nu = (int64_t)R * GW / 4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nz + nu;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const float *src;
    int64_t stride;
    int cnt;
    if (idx < nz) {
      const int64_t e = idx * 4, n = e / R;
      const int r = (int)(e - n * R);
      src = dzp + n * RP + r; stride = N * RP; cnt = ncb;
    } else {
      const int64_t o = (idx - nz) * 4;
      const int64_t r = o / GW, col = o - r * GW;
      src = dUp + r * GW + col; stride = (int64_t)RP * GW; cnt = nparts;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 8 <= cnt; c += 8) {
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4 *>(src + (c + i) * stride);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[0] += v[i][0];
        acc[1] += v[i][1];
        acc[2] += v[i][2];
        acc[3] += v[i][3];
      }
    }
    for (; c < cnt; ++c) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src + c * stride);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    if constexpr (sizeof(E) == 2) {
      const uint2 b = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      if (idx < nz) *reinterpret_cast<uint2 *>(dz + idx * 4) = b;
      else *reinterpret_cast<uint2 *>(dU + (idx - nz) * 4) = b;
    } else {
      if (idx < nz) *reinterpret_cast<f32x4 *>(dz + idx * 4) = acc;
      else *reinterpret_cast<f32x4 *>(dU + (idx - nz) * 4) = acc;
    }
  }
}
}  // namespace dsc
