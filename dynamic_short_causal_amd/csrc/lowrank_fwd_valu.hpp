// lowrank_fwd_valu.hpp -- low-rank forward on the vector ALUs for filters tied
// over H = 8 channels in bf16 (one filter group per 16-byte channel vector).
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (Mechanisme;
// Parametrisatie 1 and 2, low rank R with heads tied over H channels;
// Plaatsing, residual) and Efficiente Trainingsimplementatie, bullet "Fused
// Low-Rank Kernel": w[t,g,k] = sum_r z[t,r] U[r, g*W+k] is formed on chip and
// used at once.
//
// Why not MFMA here.  With H = 8 a channel vector is one group, so a token
// needs W filter values per vector and the contraction over the ranks is
// R*W/8 multiply-adds per channel (8 at R = 16, W = 4), an eighth of the
// per-channel case.  v_dot2_f32_bf16 takes two ranks per instruction (the
// products are exact bf16 x bf16 products summed in fp32, as on the matrix
// cores), so the filters cost W*R/2 instructions per lane and token, and
// the lane layout needs no LDS and no transposition: lane = one channel
// vector, walking the tokens of a chunk with its causal window in registers.
// The MFMA kernel (lowrank_impl.hpp) moves every token row through LDS to
// reach the matrix-core layout; at the linear-RNN shape this kernel measured
// faster.
//
// z is uniform across the wave (one token at a time), so its rank pairs are
// scalar loads; U's rank pairs of the lane's group stay in registers.
#pragma once
#include "dsc_device.hpp"
#include "lowrank_impl.hpp"

namespace dsc {

constexpr int kLvRanks = 16;  // ranks served (pairs held in registers)

// Tokens per workgroup chunk of the vector-ALU forward.  At the linear-RNN
// shape (B=16 T=4096 D=4608 W=4) 16 measured 238 us against 243 for 32, 271
// for 64 and 288 for 128: more, shorter chunks keep more waves in flight,
// and the U rows a chunk loads first cost little once each rank row is one
// 8-byte load (with 2-byte loads, 32-token chunks took 258 us).
constexpr int kLvChunk = 16;

template <int W, bool ACT, bool VL>
__global__ __launch_bounds__(256) void lr_fwd_valu_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ z, const bf16 *__restrict__ U,
    const int32_t *__restrict__ pos, bf16 *__restrict__ y, int T, int D, int R, int TC,
    int nchunk, int nvb, float rho) {
  constexpr int UN = W >= 2 ? W : 4;  // tokens per iteration: window slots repeat every W
  constexpr int RH = kLvRanks / 2;    // rank pairs
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int nvec = D / 8;
  const int v = vb * (int)blockDim.x + (int)threadIdx.x;
  const bool on = v < nvec;
  const int g = on ? v : nvec - 1;  // the lane's group (H = 8: one per vector)
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int64_t seq = (int64_t)b * T;
  const int GW = nvec * W;

  // U[r, g*W + k] for the pair (2i, 2i+1) as one bf16x2; ranks >= R are zero.
  // The W taps of a group are contiguous in a rank row: one load per row
  // (U is 16-byte aligned and its rows hold D*W/8 values, so g*W starts at a
  // multiple of the load's width).
  bf16x2_t u[RH][W];
  auto urow = [&](int r, uint32_t (&o)[W]) {  // the W taps of group g in rank row r (zero past R)
    const bf16 *p = U + (int64_t)r * GW + g * W;
    const bool ok = r < R;
    if constexpr (W == 4) {
      const uint2 v = ok ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0u, 0u);
      o[0] = v.x & 0xffffu; o[1] = v.x >> 16; o[2] = v.y & 0xffffu; o[3] = v.y >> 16;
    } else if constexpr (W == 2) {
      const uint32_t v = ok ? *reinterpret_cast<const uint32_t *>(p) : 0u;
      o[0] = v & 0xffffu; o[1] = v >> 16;
    } else {
#pragma unroll
      for (int k = 0; k < W; ++k) o[k] = ok ? (uint32_t)p[k] : 0u;
    }
  };
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    uint32_t lo[W], hi[W];
    urow(2 * i, lo);
    urow(2 * i + 1, hi);
#pragma unroll
    for (int k = 0; k < W; ++k) u[i][k] = __builtin_bit_cast(bf16x2_t, lo[k] | (hi[k] << 16));
  }

  // x rows ta .. t1-1 through a buffer resource: rows past the chunk and
  // lanes past D read zero
  const int ta = max(0, t0 - (W - 1));
  const brsrc rx = mk_rsrc(x + (seq + ta) * (int64_t)D, (int64_t)(t1 - ta) * D * 2);
  const brsrc ry = mk_rsrc(y + (seq + t0) * (int64_t)D, (int64_t)(t1 - t0) * D * 2);
  const uint32_t lo = on ? (uint32_t)v * 16 : kOOB;
  const uint32_t rowb = (uint32_t)D * 2;
  auto ldx = [&](int t) {
    return __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, lo + (uint32_t)(t - ta) * rowb, 0, kNT));
  };
  // causal window: slot (t - t0) mod W holds x[t]; taps before the sequence are zero
  float win[W][8];
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int sl = (W - k) % W;
    if (t0 - k >= 0) unpack<bf16>(ldx(t0 - k), win[sl]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) win[sl][i] = 0.f;
  }
  uint4 xc[UN];
#pragma unroll
  for (int q = 0; q < UN; ++q) xc[q] = ldx(t0 + q);

  // z rank pairs of token t (R even, so a pair never straddles two rows): the
  // pair index is clamped to the row, pairs past R/2 are zeroed where used
  const uint32_t *zbase = reinterpret_cast<const uint32_t *>(z);
  const int rp = R >> 1;
  for (int tg = t0; tg < t1; tg += UN) {
    uint4 xn[UN];
#pragma unroll
    for (int q = 0; q < UN; ++q) xn[q] = ldx(tg + UN + q);
#pragma unroll
    for (int q = 0; q < UN; ++q) {
      const int t = tg + q;
      const int sl = q % W;
      unpack<bf16>(xc[q], win[sl]);
      if (t < t1) {
        const uint32_t *zr = zbase + (((seq + t) * R) >> 1);
        uint32_t zl[RH];
#pragma unroll
        for (int i = 0; i < RH; ++i) zl[i] = zr[i < rp ? i : rp - 1];
        float w[W];
#pragma unroll
        for (int k = 0; k < W; ++k) w[k] = 0.f;
#pragma unroll
        for (int i = 0; i < RH; ++i) {
          const bf16x2_t zz = __builtin_bit_cast(bf16x2_t, i < rp ? zl[i] : 0u);
#pragma unroll
          for (int k = 0; k < W; ++k) w[k] = __builtin_amdgcn_fdot2_f32_bf16(u[i][k], zz, w[k], false);
        }
        if constexpr (VL) {  // taps reaching before the token's document are dropped
          const int pt = pos[seq + t];
#pragma unroll
          for (int k = 1; k < W; ++k)
            if (k > pt) w[k] = 0.f;
        }
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float s = 0.f;
#pragma unroll
          for (int k = 0; k < W; ++k) s = fmaf(w[k], win[(sl - k + W) % W][c], s);
          if constexpr (ACT) s = silu_f(s);
          o[c] = fmaf(rho, win[sl][c], s);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, pack<bf16>(o)), ry,
                                               lo + (uint32_t)(t - t0) * rowb, 0, kNT);
      }
    }
#pragma unroll
    for (int q = 0; q < UN; ++q) xc[q] = xn[q];
  }
}

// The vector-ALU forward serves bf16 with H = 8, W <= 4 and an even R <= 16.
// Wider windows hold 2W rows of x in flight besides the window and U (about
// 200 VGPRs at W = 8, two waves per SIMD) and stay on the MFMA kernel.  The
// buffer offsets span a chunk plus its halo and prefetch (under 64 rows),
// which must stay below 2^31 bytes.
inline bool lr_fwd_uses_valu(bool bf16, int64_t D, int W, int H, int R) {
  return bf16 && H == 8 && W <= 4 && R <= kLvRanks && (R & 1) == 0 &&
         D * 2 * 64 < ((int64_t)1 << 31);
}

template <int W, bool ACT, bool VL>
static hipError_t launch_lr_fwd_valu(const LrArgs &a) {
  const int nvec = (int)(a.D / 8);
  const int nw = (nvec + 63) / 64;  // waves needed to cover the vectors of a row
  // waves per workgroup: 4, 3 or 2, whichever leaves the fewest idle lanes
  int wpb = 4;
  for (int c : {4, 3, 2})
    if ((nw + c - 1) / c * c - nw < (nw + wpb - 1) / wpb * wpb - nw) wpb = c;
  const int bs = 64 * wpb, nvb = (nvec + bs - 1) / bs;
  const int TC = kLvChunk, nchunk = (int)((a.T + TC - 1) / TC);
  const int64_t nblocks = a.B * nchunk * (int64_t)nvb;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL((lr_fwd_valu_kernel<W, ACT, VL>), dim3((unsigned)nblocks), dim3(bs), 0,
                     (hipStream_t)a.stream, (const bf16 *)a.x, (const bf16 *)a.z,
                     (const bf16 *)a.U, a.pos, (bf16 *)a.y, (int)a.T, (int)a.D, a.R, TC, nchunk,
                     nvb, a.residual ? 1.f : 0.f);
  return hipGetLastError();
}

}  // namespace dsc
