// lowrank_fwd_cl.hpp -- low-rank forward for per-channel filters (H = 1,
// bf16, plain rows, R <= 16), one channel per lane.
//
// Operation: the low-rank dynamic short convolution (gist.science summary
// "Dynamische Korte Convoluties Verbeteren Transformers", Methodologie >
// Dynamische Korte Convoluties, Parametrisatie 1, and Efficiente
// Trainingsimplementatie, bullet "Fused Low-Rank Kernel"):
//   w[t,c,k] = sum_r z[t,r] U[r, c*W + k],
//   y[t,c] = act(sum_k w[t,c,k] x[t-k,c]) + rho x[t,c],
// with w formed on chip and never written to memory.
//
// Layout: that of the channel-per-lane backward (lowrank_bwd_cl.hpp).  A
// workgroup of 4 waves owns 128 channels and a chunk of tokens and walks it in
// 16-token steps; each wave owns two groups of 16 channels, and in a group
// lane (q, n) owns channel n and tokens 4q..4q+3 of the step.  That is the
// output layout of a 16x16 MFMA with A = z (rows = the step's tokens, K =
// ranks) and B = U (K = ranks, columns = the group's channels, one MFMA per
// tap), so every lane gets the W filter taps of its own channel and tokens
// straight from the matrix cores.  The x values of its channel at those
// tokens and the W-1 before them come from a bf16 LDS ring through the
// transposing LDS read (ds_read_b64_tr_b16: four token rows of one channel
// into one lane).  y goes back through a 16-row LDS staging tile and is
// stored in whole rows.
#pragma once
#include "lowrank_bwd_cl.hpp"

namespace dsc {

template <int W> struct LrFwdClGeo {
  static constexpr int XP = kClCB * 2 + 32;  // bf16 row pitch (x ring, y staging)
  static constexpr int ZP = 40;              // z ring row: 16 ranks + 8 bytes
  static constexpr int NHQ = (W + 2) / 4;    // x quads before the lane's own four tokens
  static constexpr int o_x = 0;
  static constexpr int o_y = o_x + 32 * XP;
  static constexpr int o_z = o_y + 16 * XP;
  static constexpr int bytes = o_z + 32 * ZP;
};

template <int W, bool ACT, int PF>
__global__ __launch_bounds__(kClThreads) void lr_fwd_cl_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ z, const bf16 *__restrict__ U,
    bf16 *__restrict__ y, int T, int D, int R, int TC, int nchunk, int ncb, float rho) {
  using Gc = LrFwdClGeo<W>;
  constexpr int XP = Gc::XP, ZP = Gc::ZP, NHQ = Gc::NHQ, NG = kClNG, VPR = kClVPR;
  static_assert(kClThreads == 16 * VPR, "one x vector of a 16-row slab per thread");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *xring = smem + Gc::o_x, *yst = smem + Gc::o_y, *zring = smem + Gc::o_z;

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int64_t seq = (int64_t)b * T;
  const int GW = D * W;  // U columns (one filter per channel)
  int cl0[NG];
#pragma unroll
  for (int u = 0; u < NG; ++u) cl0[u] = (wave * NG + u) * 16;

  // coop role: vector cv of row cr of a 16-row slab
  const int cr = tid / VPR, cv = tid % VPR;
  const int cc = cb * kClCB + cv * 8;
  const uint32_t coff = (cc < D ? (uint32_t)cc * 2 : kOOB) + (uint32_t)(cr * D * 2);
  const bool z_on = tid < 16 * R;
  const uint32_t zoff = z_on ? (uint32_t)tid * 2 : kOOB;
  const int zr_tok = tid / (R > 0 ? R : 1), zr_rank = tid - zr_tok * (R > 0 ? R : 1);
  auto slab = [&](const bf16 *base, int t, int lim, int width) {
    return mk_rsrc(base + (seq + t) * (int64_t)width, (int64_t)(min(lim, t + 16) - t) * width * 2);
  };

  // ranks past R stay zero in the z ring
  for (int i = tid; i < 32 * ZP / 4; i += kClThreads) reinterpret_cast<uint32_t *>(zring)[i] = 0u;

  // B operand per group u and tap k, lane (q, n): U[ranks 4q..4q+3][c*W + k]
  // (c = its channel); row r of U holds the W taps of channel c contiguously
  s16x4 bu[NG][W];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int c = cb * kClCB + cl0[u] + n;
    short tb[4][W];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * q + e;
      load_shorts<W>(U + (int64_t)r * GW + (int64_t)c * W, c < D && r < R, tb[e]);
    }
#pragma unroll
    for (int k = 0; k < W; ++k) bu[u][k] = s16x4{tb[0][k], tb[1][k], tb[2][k], tb[3][k]};
  }

  const int tiles = (t1 - t0 + 15) / 16;
  __syncthreads();
  {  // x of the 16 tokens before the chunk (zero before the sequence)
    const int tb = t0 - 16;
    const brsrc rx = slab(x, tb, tb < 0 ? tb : T, D);
    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, coff, 0, kNT));
    *reinterpret_cast<uint4 *>(xring + ((tb + cr) & 31) * XP + cv * 16) = v;
  }
  auto tra = [&](const unsigned char *base, int row, int col0) {
    return base + row * XP + (col0 + 4 * (n & 3)) * 2;
  };

  // the loads of step st are issued PF steps ahead, into register slot st % PF
  // (compile-time after unrolling the step loop by PF)
  uint4 xn[PF];
  bf16 zn[PF];
  auto issue = [&](int st, int sl) {
    const int t = t0 + 16 * st;
    const brsrc rz = slab(z, t, T, R);
    zn[sl] = (bf16)__builtin_amdgcn_raw_buffer_load_b16(rz, zoff, 0, 0);
    const brsrc rx = slab(x, t, T, D);
    xn[sl] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, coff, 0, kNT));
  };
  auto fill = [&](int st, int sl) {
    const int t = t0 + 16 * st;
    *reinterpret_cast<uint4 *>(xring + ((t + cr) & 31) * XP + cv * 16) = xn[sl];
    if (z_on) reinterpret_cast<bf16 *>(zring + ((t + zr_tok) & 31) * ZP)[zr_rank] = zn[sl];
  };
  // y of step st from the staging tile, in whole rows (rows past t1 dropped)
  auto flush = [&](int st) {
    const int t = t0 + 16 * st;
    const brsrc ry = slab(y, t, t1, D);
    const uint4 v = *reinterpret_cast<const uint4 *>(yst + cr * XP + cv * 16);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ry, coff, 0, kNT);
  };

  constexpr int X0 = 4 * NHQ;
  auto step = [&](int st, int sl) {
    const int t = t0 + 16 * st;
    fill(st, sl);
    if (st > 0) flush(st - 1);
    if (st + PF < tiles) issue(st + PF, sl);
    __syncthreads();  // (1) ring rows of this step written; staging of the last step read
    // A operand: row n = token t+n, ranks 4q..4q+3
    const s16x4 az = *reinterpret_cast<const s16x4 *>(zring + ((t + n) & 31) * ZP + 8 * q);
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      // xw[4h + e] = x of this lane's channel at token t + 4q - 4*NHQ + 4h + e
      float xw[4 * NHQ + 4];
#pragma unroll
      for (int h = 0; h <= NHQ; ++h) {
        const int row = (t + 4 * q - 4 * NHQ + 4 * h + (n >> 2)) & 31;
        const s16x4 xv = tr16(tra(xring, row, cl0[u]));
#pragma unroll
        for (int e = 0; e < 4; ++e) xw[4 * h + e] = bf2f(xv[e]);
      }
      float o[4];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const f32x4 wk = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(az, bu[u][k], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = k == 0 ? wk[e] * xw[X0 + e] : fmaf(wk[e], xw[X0 + e - k], o[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = o[e];
        if constexpr (ACT) s = silu_f(s);
        s = fmaf(rho, xw[X0 + e], s);
        *reinterpret_cast<uint16_t *>(yst + (4 * q + e) * XP + (cl0[u] + n) * 2) =
            __builtin_bit_cast(uint16_t, (__bf16)s);
      }
    }
    __syncthreads();  // (2) staging written, ring reads of this step done
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < tiles) issue(p, p);
  for (int s0 = 0; s0 < tiles; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (s0 + p < tiles) step(s0 + p, p);
  }
  if (tiles > 0) flush(tiles - 1);
}

}  // namespace dsc
