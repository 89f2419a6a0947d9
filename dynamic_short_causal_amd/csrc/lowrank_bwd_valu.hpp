// lowrank_bwd_valu.hpp -- low-rank backward on the vector ALUs for bf16
// filters tied over H = 8 channels (one filter group per 16-byte channel
// vector), the layout of the vector-ALU forward (lowrank_fwd_valu.hpp).
//
// Operation: the derivative of the low-rank dynamic short convolution
// (gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties, Parametrisatie
// 1 and 2; Efficiente Trainingsimplementatie, bullet "Fused Low-Rank Kernel"):
//   ds = dy * act'(s),  dx[t] = rho dy[t] + sum_k w[t+k,.,k] ds[t+k],
//   dw[t,g,k] = sum_{c in g} ds[t,c] x[t-k,c],  dz = dw U^T,  dU = z^T dw.
//
// A lane owns one channel vector (= one group) and walks the tokens of a
// chunk plus the W-1 tokens after it:
//   * the filters of token t from v_dot2_f32_bf16 over rank pairs of U held
//     in registers, z as scalar loads;
//   * dx by scattering w[t,k] ds[t] into the accumulators of tokens t-k
//     (W slots, one completed per token);
//   * dw of the lane's group is a sum over its own 8 channels;
//   * dU[r, g*W+k] += z[t,r] dw[t,k] in R*W fp32 registers per lane,
//     written once per chunk as a partial;
//   * dz[t,r] = sum_{g,k} dw U: each lane's 16 products are summed across
//     the wave by a transposing reduction (permlane swaps at lane distances 32
//     and 16, row rotations below), across the waves of the workgroup in
//     LDS, and written as one fp32 partial per workgroup and token.
// The partials have the layout lr_reduce_kernel adds (dz [block][B*T][16],
// dU [B*chunks][16][G*W]).
#pragma once
#include "dsc_device.hpp"
#include "lowrank_impl.hpp"
#include "lowrank_fwd_valu.hpp"

namespace dsc {

constexpr int kLbChunk = 256;  // tokens per chunk of the vector-ALU backward
constexpr int kLbTB = 16;      // tokens per dz batch (one workgroup barrier)

// Sum of v[0..15] over the 64 lanes of the wave.  On return lane l holds the
// total of value l >> 2 (every lane of a quad the same).
__device__ __forceinline__ float wave_sum16(float (&v)[16], int lane) {
  float a[8];
  // lane distance 32: the low half keeps values 0..7, the high half 8..15
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]),
                                                    false, false);
    a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // lane distance 16 (rows): even rows keep 0..3, odd rows 4..7 of a
  float b4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 4]),
                                                    false, false);
    b4[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // lane distance 8 inside a row (rotation by 8): lanes with bit 3 clear keep
  // b4[0..1], the others b4[2..3]
  const bool h8 = (lane >> 3) & 1;
  float c2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = h8 ? b4[i + 2] : b4[i];
    const float send = h8 ? b4[i] : b4[i + 2];
    c2[i] = keep + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(send), 0x128, 0xf,
                                                                0xf, false));
  }
  // lane distance 4 (mirror inside each half row: lane i <-> 7 - i flips bit 2)
  const bool h4 = (lane >> 2) & 1;
  const float keep = h4 ? c2[1] : c2[0];
  const float send = h4 ? c2[0] : c2[1];
  float d = keep + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(send), 0x141, 0xf,
                                                                0xf, false));
  // the four lanes of a quad hold partial sums of the same value
  d += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(d), 0x4E, 0xf, 0xf, false));
  d += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(d), 0xB1, 0xf, 0xf, false));
  return d;
}

// Partial-sum layout of one vector-ALU backward call.
struct LbPlan {
  int wpb, bs, nvb, nchunk;
  size_t dz_part, dU_part, bytes;
};

inline LbPlan lr_bwd_valu_plan(int64_t B, int64_t T, int64_t D, int W) {
  LbPlan p{};
  const int nvec = (int)(D / 8);
  const int nw = (nvec + 63) / 64;
  p.wpb = 4;
  for (int c : {4, 3, 2})
    if ((nw + c - 1) / c * c - nw < (nw + p.wpb - 1) / p.wpb * p.wpb - nw) p.wpb = c;
  p.bs = 64 * p.wpb;
  p.nvb = (nvec + p.bs - 1) / p.bs;
  p.nchunk = (int)((T + kLbChunk - 1) / kLbChunk);
  p.dz_part = (size_t)p.nvb * (size_t)(B * T) * 16 * 4;
  p.dU_part = (size_t)(B * p.nchunk) * 16 * (size_t)(nvec * W) * 4;
  p.bytes = p.dz_part + p.dU_part;
  return p;
}

template <int W, bool ACT>
__global__ __launch_bounds__(256, 2) void lr_bwd_valu_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ z, const bf16 *__restrict__ U,
    const bf16 *__restrict__ dy, bf16 *__restrict__ dx, float *__restrict__ dzp,
    float *__restrict__ dUp, int T, int D, int R, int nchunk, int nvb, int64_t N, float rho) {
  constexpr int UN = W >= 2 ? W : 4;  // tokens per group: slots repeat every W tokens
  constexpr int RH = kLvRanks / 2;
  __shared__ float dzl[2][kLbTB][4][16];  // per batch: token, wave, rank
  int bid = blockIdx.x;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwv = blockDim.x >> 6;
  const int nvec = D / 8;
  const int v = vb * (int)blockDim.x + tid;
  const bool on = v < nvec;
  const int g = on ? v : nvec - 1;
  const int t0 = chunk * kLbChunk, t1 = min(T, t0 + kLbChunk);
  const int te = t1 + W - 1;  // tokens t1 .. te-1 only complete dx (past T: zero)
  const int64_t seq = (int64_t)b * T;
  const int GW = nvec * W;

  bf16x2_t u[RH][W];
#pragma unroll
  for (int i = 0; i < RH; ++i)
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const uint32_t lo = 2 * i < R ? (uint32_t)U[(int64_t)(2 * i) * GW + g * W + k] : 0u;
      const uint32_t hi = 2 * i + 1 < R ? (uint32_t)U[(int64_t)(2 * i + 1) * GW + g * W + k] : 0u;
      u[i][k] = __builtin_bit_cast(bf16x2_t, lo | (hi << 16));
    }

  const int ta = max(0, t0 - (W - 1));
  const int tx = min(T, te);  // rows of x and dy that exist
  const brsrc rx = mk_rsrc(x + (seq + ta) * (int64_t)D, (int64_t)(tx - ta) * D * 2);
  const brsrc rdy = mk_rsrc(dy + (seq + t0) * (int64_t)D, (int64_t)(tx - t0) * D * 2);
  const brsrc rdx = mk_rsrc(dx + (seq + t0) * (int64_t)D, (int64_t)(t1 - t0) * D * 2);
  const uint32_t lo = on ? (uint32_t)v * 16 : kOOB;
  const uint32_t rowb = (uint32_t)D * 2;
  auto ldx = [&](int t) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, lo + (uint32_t)(t - ta) * rowb, 0, kNT));
  };
  auto lddy = [&](int t) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rdy, lo + (uint32_t)(t - t0) * rowb, 0, kNT));
  };

  float win[W][8];  // slot (t - t0) mod W holds x[t]
#pragma unroll
  for (int k = 1; k < W; ++k) {
    const int sl = (W - k) % W;
    if (t0 - k >= 0) unpack<bf16>(ldx(t0 - k), win[sl]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) win[sl][i] = 0.f;
  }
  float dxa[W][8];  // slot (t - t0) mod W: dx of token t so far
#pragma unroll
  for (int k = 0; k < W; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) dxa[k][i] = 0.f;
  float dUa[2 * RH][W];
#pragma unroll
  for (int r = 0; r < 2 * RH; ++r)
#pragma unroll
    for (int k = 0; k < W; ++k) dUa[r][k] = 0.f;

  const uint32_t *zbase = reinterpret_cast<const uint32_t *>(z);
  const int rp = R >> 1;
  uint4 xc[UN], dyc[UN];
#pragma unroll
  for (int q = 0; q < UN; ++q) {
    xc[q] = ldx(t0 + q);
    dyc[q] = lddy(t0 + q);
  }
  // x and dy rows of token t sit in slot (t - t0) mod UN of xc, dyc and are
  // replaced by the rows of token t + UN as soon as they are unpacked
  for (int tg = t0; tg < te; tg += UN) {
#pragma unroll
    for (int q = 0; q < UN; ++q) {
      const int t = tg + q;
      const int sl = q % W;
      unpack<bf16>(xc[q], win[sl]);
      float dyv[8];
      unpack<bf16>(dyc[q], dyv);
      xc[q] = ldx(t + UN);
      dyc[q] = lddy(t + UN);
      if (t < te) {
        // filters of token t (z of the last token for tokens past T: ds is zero there)
        const uint32_t *zr = zbase + (((seq + min(t, T - 1)) * R) >> 1);
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
        float ds[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if constexpr (ACT) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < W; ++k) s = fmaf(w[k], win[(sl - k + W) % W][c], s);
            ds[c] = dyv[c] * silu_grad_f(s);
          } else {
            ds[c] = dyv[c];
          }
        }
        // dx: token t adds w[t,k] ds[t] to token t-k, and rho dy[t] to itself
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
          for (int c = 0; c < 8; ++c) dxa[(sl - k + W) % W][c] = fmaf(w[k], ds[c], dxa[(sl - k + W) % W][c]);
#pragma unroll
        for (int c = 0; c < 8; ++c) dxa[sl][c] = fmaf(rho, dyv[c], dxa[sl][c]);
        if (t < t1) {
          // filter gradient of the lane's group
          float dw[W];
#pragma unroll
          for (int k = 0; k < W; ++k) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) a = fmaf(ds[c], win[(sl - k + W) % W][c], a);
            dw[k] = a;
          }
          // dU += z dw (z in fp32, from the scalar pairs)
#pragma unroll
          for (int i = 0; i < RH; ++i) {
            const uint32_t zz = i < rp ? zl[i] : 0u;
            const float z0 = __uint_as_float(zz << 16), z1 = __uint_as_float(zz & 0xffff0000u);
#pragma unroll
            for (int k = 0; k < W; ++k) {
              dUa[2 * i][k] = fmaf(z0, dw[k], dUa[2 * i][k]);
              dUa[2 * i + 1][k] = fmaf(z1, dw[k], dUa[2 * i + 1][k]);
            }
          }
          // dz: the lane's products for the 16 ranks (dw rounded to bf16, as
          // the matrix-core kernels round it), summed over the wave
          float dzv[2 * RH];
#pragma unroll
          for (int r = 0; r < 2 * RH; ++r) dzv[r] = 0.f;
#pragma unroll
          for (int k = 0; k < W; ++k) {
            const uint32_t dwb = pack_bf16x2(dw[k], 0.f) & 0xffffu;
            const bf16x2_t dlo = __builtin_bit_cast(bf16x2_t, dwb);
            const bf16x2_t dhi = __builtin_bit_cast(bf16x2_t, dwb << 16);
#pragma unroll
            for (int i = 0; i < RH; ++i) {
              dzv[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(u[i][k], dlo, dzv[2 * i], false);
              dzv[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(u[i][k], dhi, dzv[2 * i + 1], false);
            }
          }
          if (!on)
#pragma unroll
            for (int r = 0; r < 2 * RH; ++r) dzv[r] = 0.f;
          const float tot = wave_sum16(dzv, lane);
          const int tb = (t - t0) & (kLbTB - 1), buf = ((t - t0) / kLbTB) & 1;
          if ((lane & 3) == 0) dzl[buf][tb][wave][lane >> 2] = tot;
          // end of a batch (or of the chunk): the workgroup adds its waves
          if (tb == kLbTB - 1 || t == t1 - 1) {
            __syncthreads();
            const int tbase = t - tb;
            for (int i = tid; i < (tb + 1) * 16; i += blockDim.x) {
              const int tt = i >> 4, r = i & 15;
              float sacc = dzl[buf][tt][0][r];
              for (int w2 = 1; w2 < nwv; ++w2) sacc += dzl[buf][tt][w2][r];
              dzp[((int64_t)vb * N + seq + tbase + tt) * 16 + r] = sacc;
            }
          }
        }
        // token t-W+1 is complete
        const int td = t - (W - 1);
        const int sd = (sl + 1) % W;
        if (td >= t0 && td < t1)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, pack<bf16>(dxa[sd])), rdx,
                                                 lo + (uint32_t)(td - t0) * rowb, 0, kNT);
#pragma unroll
        for (int c = 0; c < 8; ++c) dxa[sd][c] = 0.f;
      }
    }
  }
  // dU partial of this chunk: rank r, the lane's W columns
  if (on) {
    float *dst = dUp + (int64_t)(b * nchunk + chunk) * 16 * GW + (int64_t)g * W;
#pragma unroll
    for (int r = 0; r < 2 * RH; ++r) store_floats<W>(dst + (int64_t)r * GW, dUa[r]);
  }
}

// The vector-ALU backward serves what the vector-ALU forward serves, without
// packed rows.
inline bool lr_bwd_uses_valu(bool bf16, int64_t D, int W, int H, int R, bool vl) {
  return !vl && lr_fwd_uses_valu(bf16, D, W, H, R) && D * 2 * (kLbChunk + 16) < ((int64_t)1 << 31);
}

template <int W, bool ACT>
static hipError_t launch_lr_bwd_valu(const LrArgs &a, float *dzp, float *dUp) {
  const LbPlan p = lr_bwd_valu_plan(a.B, a.T, a.D, W);
  const int64_t nblocks = a.B * p.nchunk * (int64_t)p.nvb;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL((lr_bwd_valu_kernel<W, ACT>), dim3((unsigned)nblocks), dim3(p.bs), 0,
                     (hipStream_t)a.stream, (const bf16 *)a.x, (const bf16 *)a.z,
                     (const bf16 *)a.U, (const bf16 *)a.dy, (bf16 *)a.dx, dzp, dUp, (int)a.T,
                     (int)a.D, a.R, p.nchunk, p.nvb, a.B * a.T, a.residual ? 1.f : 0.f);
  return hipGetLastError();
}

}  // namespace dsc
