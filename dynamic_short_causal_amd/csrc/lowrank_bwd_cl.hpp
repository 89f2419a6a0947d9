// lowrank_bwd_cl.hpp -- low-rank backward for per-channel filters (H = 1,
// bf16, no activation), one channel per lane.
//
// Operation: the derivative of the low-rank dynamic short convolution (gist.science
// summary "Dynamische Korte Convoluties Verbeteren Transformers", Methodologie >
// Dynamische Korte Convoluties, Parametrisatie 1, and Efficiente
// Trainingsimplementatie, bullet "Fused Low-Rank Kernel"):
//   ds = dy,  dx[t] = rho dy[t] + sum_k w[t+k,.,k] ds[t+k],
//   dw[t,c,k] = ds[t,c] x[t-k,c],  dz = dw U^T,  dU = z^T dw.
//
// Layout.  A workgroup of 4 waves owns 128 channels and a chunk of tokens and
// walks it in 16-token steps.  Each wave owns two groups of 16 channels.  In a
// group, lane (q, n) (q = lane / 16, n = lane % 16) owns channel n and the four
// consecutive tokens 4q..4q+3 of the step: exactly the output layout of a 16x16
// MFMA whose rows are tokens and whose columns are channels.  So
//   * filters come from MFMAs with A = z (rows = tokens, K = ranks) and
//     B = U (K = ranks, columns = this group's channels), one per tap; for dx
//     the A rows are z of tokens t+k ("shifted filters");
//   * the causal taps of the lane's own tokens are in its registers; x and ds
//     of the neighbouring tokens come from LDS;
//   * dU[rank][channel] += z^T dw needs no transpose: the lane's four dw values
//     (K = its four tokens) are the B operand as they stand;
//   * dz^T = U dw^T contracts over channels, so dw goes through LDS once, read
//     back with the transposing LDS read (ds_read_b64_tr_b16);
//   * x and dy come from LDS slabs filled by row-major loads, read with the
//     transposing read, which turns four token rows of one channel into one
//     lane's four values.
// Compared with one token per lane, each element costs about half the vector-
// ALU instructions and LDS bytes; at the QKV shape it measured 187 against
// 234 us when this dispatch was chosen (152.6 us in the current trace).  Tied
// heads (H > 1) turn every channel into a filter slot (H times the dz/dU MFMA
// work of per-group slots), and the SiLU recomputation needs a second set of
// filter MFMAs and registers that drop the kernel to two waves per SIMD;
// measured at the QKV shape, the token-per-lane kernel is as fast or faster
// in both cases (H = 1 with SiLU: 269 against 320 us), so they use it.
//
// Rows past the sequence are handled by buffer resources (read as zero, not
// written); the partials of dz (per channel block) and dU (per chunk) are the
// same as those of the token-per-lane kernel and are reduced by the same
// kernel.
#pragma once
#include "lowrank_impl.hpp"

namespace dsc {

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
// Transposing LDS read (gfx950): in each 16-lane group, lane l receives element
// l % 4 of the 8-byte chunks addressed by lanes 4e + l / 4, e = 0..3.  When lane
// s addresses the chunk (row r0 + s/4, columns c0 + 4(s%4) .. +3) of a 16-bit
// row-major array, lane l receives column c0 + l of rows r0 .. r0+3.
__device__ __forceinline__ s16x4 tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t *)(__attribute__((address_space(3))) char *)(uintptr_t)p);
}
// bf16 bits -> float
__device__ __forceinline__ float bf2f(short v) { return __uint_as_float((uint32_t)(uint16_t)v << 16); }

// N consecutive 16-bit values from p (zeros when !ok), with the widest loads
// the alignment of p allows (p is aligned to 2N bytes rounded down to a power
// of two, up to 16, at every call site)
template <int N>
__device__ __forceinline__ void load_shorts(const bf16 *p, bool ok, short (&o)[N]) {
  constexpr int B = (N % 8 == 0) ? 8 : (N % 4 == 0) ? 4 : (N % 2 == 0) ? 2 : 1;
#pragma unroll
  for (int i = 0; i < N; i += B) {
    if constexpr (B == 8) {
      const uint4 v = ok ? *reinterpret_cast<const uint4 *>(p + i) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) o[i + j] = (short)(w[j >> 1] >> (16 * (j & 1)));
    } else if constexpr (B == 4) {
      const uint2 v = ok ? *reinterpret_cast<const uint2 *>(p + i) : make_uint2(0u, 0u);
      const uint32_t w[2] = {v.x, v.y};
#pragma unroll
      for (int j = 0; j < 4; ++j) o[i + j] = (short)(w[j >> 1] >> (16 * (j & 1)));
    } else if constexpr (B == 2) {
      const uint32_t v = ok ? *reinterpret_cast<const uint32_t *>(p + i) : 0u;
      o[i] = (short)v;
      o[i + 1] = (short)(v >> 16);
    } else {
      o[i] = ok ? (short)p[i] : (short)0;
    }
  }
}
template <int N>
__device__ __forceinline__ void store_floats(float *p, const float (&v)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<f32x4 *>(p + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = v[i];
  }
}

constexpr int kClWaves = kLrClWaves;           // waves per workgroup
constexpr int kClNG = kLrClNG;                 // 16-channel groups per wave
constexpr int kClThreads = 64 * kClWaves;
constexpr int kClCB = kLrClCB;                 // channels per workgroup
constexpr int kClVPR = kClCB / 8;              // 16-byte vectors per row of the block
// every thread moves one vector of x and one of dy per step, or (with twice as
// many threads as vectors of a 16-row slab) one vector of either
constexpr bool kClSplit = kClThreads == 32 * kClVPR;
static_assert(kClSplit || kClThreads == 16 * kClVPR, "one or two slab vectors per thread");

template <int W> struct LrBwdClGeo {
  static constexpr int XP = kClCB * 2 + 32;    // bf16 row pitch (x and dy rings, dx staging)
  static constexpr int ZP = 40;                // z ring row: 16 ranks + 8 bytes
  static constexpr int NHQ = (W + 2) / 4;      // x halo quads
  static constexpr int NDQ = (W + 6) / 4;      // dy quads for dx
  static constexpr int CHK = W * 64 * 8;       // dw chunks of one wave and group
  static constexpr int o_x = 0;
  static constexpr int o_dy = o_x + 32 * XP;
  static constexpr int o_dx = o_dy + 32 * XP;
  static constexpr int o_z = o_dx + 16 * XP;
  static constexpr int o_chk = o_z + 32 * ZP;
  static constexpr int o_dz = o_chk + kClWaves * CHK;
  static constexpr int o_pos = o_dz + kClWaves * 64 * 16;  // 32 document positions (VL)
  static constexpr int bytes = o_pos + 32 * 4;
};

// Waves per SIMD: as many as the compiler fits without spilling (read off the
// kernel resource-usage report; the register count grows with W).
template <int W, bool VL>
constexpr int lr_bwd_cl_min_waves() {
  // the position masks of packed rows tip W = 4, 7 and 8 over
  if constexpr (W == 8 || (VL && W == 7)) return 1;
  if constexpr (VL && W == 4) return 2;
  return W <= 4 ? 3 : 2;
}

// Packed rows (VL): a 32-entry ring of document positions.  A tap k >= 1 of a
// token beyond its position is dropped: for dx by zeroing that token's z row
// in the tap-k A operand (one row per lane), for dw by a per-lane bit mask
// over (own token, tap), so dz and dU follow.
template <int W, bool VL>
__global__ __launch_bounds__(kClThreads, (lr_bwd_cl_min_waves<W, VL>())) void lr_bwd_cl_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ z, const bf16 *__restrict__ U,
    const bf16 *__restrict__ dy, const int32_t *__restrict__ pos, bf16 *__restrict__ dx,
    float *__restrict__ dzp, float *__restrict__ dUp, int T, int D, int R, int TC, int nchunk,
    int ncb, int64_t N, float rho) {
  using Gc = LrBwdClGeo<W>;
  constexpr int XP = Gc::XP, ZP = Gc::ZP, NHQ = Gc::NHQ, NDQ = Gc::NDQ, NG = kClNG;
  constexpr int RP = 16, VPR = kClVPR;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *xring = smem + Gc::o_x, *dyring = smem + Gc::o_dy, *dxst = smem + Gc::o_dx,
                *zring = smem + Gc::o_z;
  float *dzbuf = reinterpret_cast<float *>(smem + Gc::o_dz);
  int *pring = reinterpret_cast<int *>(smem + Gc::o_pos);

  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned char *chk = smem + Gc::o_chk + wave * Gc::CHK;
  int bid = blockIdx.x;
  const int cb = bid % ncb;
  bid /= ncb;
  const int chunk = bid % nchunk;
  const int b = bid / nchunk;
  const int t0 = chunk * TC, t1 = min(T, t0 + TC);
  const int64_t seq = (int64_t)b * T;
  const int GW = D * W;  // U columns (one filter per channel)
  // group u of this wave: channels cl0[u] + n of the block
  int cl0[NG];
  bool cok[NG];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    cl0[u] = (wave * NG + u) * 16;
    cok[u] = cb * kClCB + cl0[u] + n < D;
  }

  // coop role: vector cv of row cr of a 16-row slab; with kClSplit the first
  // half of the threads moves x and the second half dy
  const int cidx = kClSplit ? tid % (16 * VPR) : tid;
  const bool c_x = !kClSplit || tid < 16 * VPR, c_dy = !kClSplit || tid >= 16 * VPR;
  const int cr = cidx / VPR, cv = cidx % VPR;
  const int cc = cb * kClCB + cv * 8;
  const uint32_t coff = (cc < D ? (uint32_t)cc * 2 : kOOB) + (uint32_t)(cr * D * 2);
  const bool z_on = tid < 16 * R;
  const uint32_t zoff = z_on ? (uint32_t)tid * 2 : kOOB;
  const int zr_tok = tid / (R > 0 ? R : 1), zr_rank = tid - zr_tok * (R > 0 ? R : 1);
  auto slab = [&](const bf16 *base, int t, int lim, int width, int pitch) {
    return mk_rsrc(base + (seq + t) * (int64_t)pitch, (int64_t)(min(lim, t + 16) - t) * width * 2);
  };

  for (int i = tid; i < 32 * ZP / 4; i += kClThreads) reinterpret_cast<uint32_t *>(zring)[i] = 0u;

  // Resident U fragments per group u and tap k:
  //  bu: filter B operand, lane (q, n): U[ranks 4q..4q+3][c*W + k] (c = its channel);
  //      row r of U holds the W taps of channel c contiguously;
  //  uz: dz A operand, lane (q, n): U[rank n][(c4+e)*W + k], e = 0..3, where
  //      c4 = the group's channel 4q: 4W contiguous values of row n.
  s16x4 bu[NG][W], uz[NG][W];
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    const int c = cb * kClCB + cl0[u] + n;
    short tb[4][W];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * q + e;
      load_shorts<W>(U + (int64_t)r * GW + (int64_t)c * W, cok[u] && r < R, tb[e]);
    }
    const int c4 = cb * kClCB + cl0[u] + 4 * q;
    short tz[4 * W];
    load_shorts<4 * W>(U + (int64_t)n * GW + (int64_t)c4 * W, c4 < D && n < R, tz);
#pragma unroll
    for (int k = 0; k < W; ++k) {
      bu[u][k] = s16x4{tb[0][k], tb[1][k], tb[2][k], tb[3][k]};
      uz[u][k] = s16x4{tz[k], tz[W + k], tz[2 * W + k], tz[3 * W + k]};
    }
  }
  f32x4 accU[NG][W];
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int k = 0; k < W; ++k) accU[u][k] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int tiles = (t1 - t0 + 15) / 16;
  __syncthreads();
  if (c_x) {  // x of the 16 tokens before the chunk (zero before the sequence)
    const int tb = t0 - 16;
    const brsrc rx = slab(x, tb, tb < 0 ? tb : T, D, D);
    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, coff, 0, kNT));
    *reinterpret_cast<uint4 *>(xring + ((tb + cr) & 31) * XP + cv * 16) = v;
  }
  // transposing-read address: rows row .. row+3 (lane quads) of columns col0 ..
  auto tra = [&](const unsigned char *base, int row, int col0) {
    return base + row * XP + (col0 + 4 * (n & 3)) * 2;
  };

  // Loads of step st are issued one step ahead, into registers.  (Two or
  // three steps ahead needed registers beyond three waves per SIMD and ran
  // slower.)  The last step (`halo`) loads only dy, z and positions: it
  // completes dx of the chunk's last tile.
  uint4 xn, dyn;
  bf16 zn;
  int pn;
  auto issue = [&](int st) {
    const int t = t0 + 16 * st;
    const bool halo = st == tiles;
    if constexpr (VL) {
      const brsrc rp = mk_rsrc(pos + seq + t, (int64_t)(min(T, t + 16) - t) * 4);
      pn = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, tid < 16 ? (uint32_t)tid * 4 : kOOB, 0, 0);
    }
    const brsrc rz = slab(z, t, T, R, R);
    zn = (bf16)__builtin_amdgcn_raw_buffer_load_b16(rz, zoff, 0, 0);
    if (c_dy) {
      const brsrc rd = slab(dy, t, T, D, D);
      dyn = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, coff, 0, kNT));
    }
    if (c_x && !halo) {
      const brsrc rx = slab(x, t, T, D, D);
      xn = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, coff, 0, kNT));
    }
  };
  auto fill = [&](int st, bool halo) {
    const int t = t0 + 16 * st;
    const int row = (t + cr) & 31;
    if (c_x && !halo) *reinterpret_cast<uint4 *>(xring + row * XP + cv * 16) = xn;
    if (c_dy) *reinterpret_cast<uint4 *>(dyring + row * XP + cv * 16) = dyn;
    if (z_on) reinterpret_cast<bf16 *>(zring + ((t + zr_tok) & 31) * ZP)[zr_rank] = zn;
    if (VL && tid < 16) pring[(t + tid) & 31] = pn;
  };

  // The device stores of step st (dx of tile st-1 from the staging rows, dz of
  // tile st summed by wave 0 in wave order; lane (q, j) holds ranks 4q..4q+3
  // of token t + j) are issued at the start of step st + 1, after its fill and
  // before its prefetch.  Stores count in the same counter as loads, so the
  // fill's wait for its prefetched rows then never waits for stores issued
  // after those loads.
  auto flush = [&](int st) {
    const int t = t0 + 16 * st;
    if (st > 0 && c_x) {
      const brsrc rdx = slab(dx, t - 16, t1, D, D);
      const uint4 v = *reinterpret_cast<const uint4 *>(dxst + cr * XP + cv * 16);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rdx, coff, 0, kNT);
    }
    if (st < tiles && wave == 0 && t + n < t1) {
      f32x4 s4 = *reinterpret_cast<const f32x4 *>(dzbuf + lane * 4);
#pragma unroll
      for (int w2 = 1; w2 < kClWaves; ++w2) s4 += *reinterpret_cast<const f32x4 *>(dzbuf + (w2 * 64 + lane) * 4);
      *reinterpret_cast<f32x4 *>(dzp + ((int64_t)cb * N + seq + t + n) * RP + 4 * q) = s4;
    }
  };
  // ds = dy, so the residual rho dy folds into the tap-0 filter; dyp holds the
  // lane's own four dy values of the step before (the first dy quad of its dx)
  const float rho_tap = rho;
  float dyp[NG][4];
  // halo_c: std::true_type for the last step (tokens after the chunk, dx
  // only).  Resolving it at compile time keeps every dU accumulation of the
  // main steps unconditional, so the accumulators stay in place across them.
  auto step = [&](int st, auto halo_c) {
    constexpr bool halo = decltype(halo_c)::value;
    const int t = t0 + 16 * st;
    fill(st, halo);
    if (st > 0) flush(st - 1);
    if (!halo) issue(st + 1);
    __syncthreads();  // (1) rings of this step written; staging and dz tiles of the last read
    constexpr int X0 = 4 * NHQ;
    float dyc[NG][4], xw[NG][4 * NHQ + 4];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const s16x4 v = tr16(tra(dyring, (t + 4 * q + (n >> 2)) & 31, cl0[u]));
#pragma unroll
      for (int e = 0; e < 4; ++e) dyc[u][e] = bf2f(v[e]);
#pragma unroll
      for (int h = 0; h <= NHQ; ++h) {
        const int row = (t + 4 * q - 4 * NHQ + 4 * h + (n >> 2)) & 31;
        const s16x4 xv = tr16(tra(xring, row, cl0[u]));
#pragma unroll
        for (int e = 0; e < 4; ++e) xw[u][4 * h + e] = bf2f(xv[e]);
      }
    }
    // bit 8e+k: tap k of the lane's own token t+4q+e lies before its
    // document (VL)
    uint32_t mown = 0;
    if constexpr (VL) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pe = pring[(t + 4 * q + e) & 31];
#pragma unroll
        for (int k = 1; k < W; ++k) mown |= (k > pe ? 1u : 0u) << (8 * e + k);
      }
    }
    auto own_off = [&](int e, int k) { return VL && k > 0 && ((mown >> (8 * e + k)) & 1u); };
    if (st > 0) {
      // dx of the previous tile: lane (q, n) forms tokens t-16+4q+e, e < 4, from
      // ds = dy at t-16+4q .. t-16+4q+4*NDQ-1 (first quad: dyp; the rest from the ring)
      s16x4 az[W];
#pragma unroll
      for (int k = 0; k < W; ++k) {
        az[k] = *reinterpret_cast<const s16x4 *>(zring + ((t - 16 + n + k) & 31) * ZP + 8 * q);
        // row n of the tap-k operand is token t-16+n+k: drop it where tap k
        // reaches before that token's document (VL)
        if (VL && k > 0 && k > pring[(t - 16 + n + k) & 31]) az[k] = s16x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        float dq[4 * NDQ];
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[e] = dyp[u][e];
#pragma unroll
        for (int h = 1; h < NDQ; ++h) {
          const s16x4 v = tr16(tra(dyring, (t - 16 + 4 * q + 4 * h + (n >> 2)) & 31, cl0[u]));
#pragma unroll
          for (int e = 0; e < 4; ++e) dq[4 * h + e] = bf2f(v[e]);
        }
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const float ini = k == 0 ? rho_tap : 0.f;
          const f32x4 wk = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(az[k], bu[u][k], f32x4{ini, ini, ini, ini}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = fmaf(wk[e], dq[e + k], o[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<uint16_t *>(dxst + (4 * q + e) * XP + (cl0[u] + n) * 2) =
              __builtin_bit_cast(uint16_t, (__bf16)o[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) dyp[u][e] = dyc[u][e];
    if constexpr (!halo) {
      const s16x4 azt = tr16(zring + ((t + 4 * q + (n >> 2)) & 31) * ZP + 8 * (n & 3));
      // chunk read by this lane; chunk c is stored at slot c ^ (bit 5 of c ->
      // bit 3), so the 32 chunks of one read pass sit on 32 distinct bank pairs
      // (a quarter fewer LDS bank-conflict cycles, no change in time measured)
      const int src = 16 * (n & 3) + 4 * q + (n >> 2);
      const int srcs = src ^ (((src >> 5) & 1) << 3), lanes = lane ^ (((lane >> 5) & 1) << 3);
      f32x4 dzacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        s16x4 bdw[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float pr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pr[e] = own_off(e, k) ? 0.f : dyc[u][e] * xw[u][X0 + e - k];
          const uint32_t p0 = pack_bf16x2(pr[0], pr[1]);
          const uint32_t p1 = pack_bf16x2(pr[2], pr[3]);
          bdw[k] = __builtin_bit_cast(s16x4, make_uint2(p0, p1));
          accU[u][k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(azt, bdw[k], accU[u][k], 0, 0, 0);
        }
        if (u > 0) __builtin_amdgcn_wave_barrier();  // previous group's chunk reads before these writes
#pragma unroll
        for (int k = 0; k < W; ++k) *reinterpret_cast<s16x4 *>(chk + (k * 64 + lanes) * 8) = bdw[k];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < W; ++k) {
          const s16x4 bt = tr16(chk + (k * 64 + srcs) * 8);
          dzacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(uz[u][k], bt, dzacc, 0, 0, 0);
        }
      }
      *reinterpret_cast<f32x4 *>(dzbuf + (wave * 64 + lane) * 4) = dzacc;
    }
    __syncthreads();  // (2) staging, dz tiles and ring reads of this step complete
  };
  issue(0);
  for (int st = 0; st < tiles; ++st) step(st, std::false_type{});
  step(tiles, std::true_type{});
  flush(tiles);
  // dU partial of this chunk: lane (q, n) holds ranks 4q..4q+3 of channel c,
  // every tap; a rank row of U has channel c's W taps contiguously
  float *dst = dUp + (int64_t)(b * nchunk + chunk) * RP * GW;
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    if (!cok[u]) continue;
    const int c = cb * kClCB + cl0[u] + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v[W];
#pragma unroll
      for (int k = 0; k < W; ++k) v[k] = accU[u][k][e];
      store_floats<W>(dst + (int64_t)(4 * q + e) * GW + (int64_t)c * W, v);
    }
  }
}
}  // namespace dsc
