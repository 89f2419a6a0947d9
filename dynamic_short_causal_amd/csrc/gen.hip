// gen.hip -- head-wise dynamic short convolution with the filters generated on
// chip from a hidden state: w[n, :] = xh[n, :] M, then y as in the head-wise
// forward.  w never reaches device memory.
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (bullets
// Mechanisme and Parametrisatie: the filter is a learned linear map of the
// hidden state; Parametrisatie 2, head-wise tying); the wispaper.ai blog
// "Dynamic Short Convolutions", Limitations, names merging the convolution into
// the preceding matrix product as the next step for inference.
//
// Mapping: a workgroup of 4 waves owns 64 tokens (flattened b*T + t) and 256
// filter columns, i.e. 256 / W groups of H channels.
//   * GEMM: the 64 x 256 tile of w = xh M accumulates over Dh in K-tiles of
//     64 staged in LDS (xh rows, M rows), with the next tile's loads held in
//     registers while the current one is consumed.  Each wave computes 64 x 64
//     with 16x16x32 bf16 MFMAs: A fragments are 16-byte row reads, B fragments
//     come from the transposing LDS read (ds_read_b64_tr_b16).
//   * Epilogue: the tile is rounded to bf16 (the precision a stored w would
//     have) into LDS; threads then walk (channel vector, token segment) items:
//     the causal window of x comes from device memory (rows of the same
//     sequence only), the taps from the LDS tile, and y goes out in 16-byte
//     stores.  A token tile may span two sequences; the window restarts at
//     every sequence start.
#include "dsc_device.hpp"
#include "gen_launch.hpp"

namespace dsc {

namespace {

typedef short s16x4g __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8g __attribute__((ext_vector_type(8)));
typedef float f32x4g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4g lds_s16x4g;

constexpr int kGenThreads = 256;
constexpr int kGT = 64;                    // tokens per workgroup
constexpr int kGC = 256;                   // filter columns per workgroup
constexpr int kGK = 64;                    // K-tile
constexpr int kAP = kGK * 2 + 16;          // A tile row pitch (bytes)
constexpr int kBP = kGC * 2 + 32;          // B tile row pitch: rows 4 apart hit distinct banks
constexpr int kWP = kGC * 2 + 16;          // w tile row pitch
constexpr int kOffB = kGT * kAP;           // B tile after the A tile
constexpr int kLdsBytes = kOffB + kGK * kBP;
static_assert(kGT * kWP <= kGK * kBP, "the w tile reuses the B tile");

__device__ __forceinline__ s16x4g tr16g(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4g *)(__attribute__((address_space(3))) char *)(uintptr_t)p);
}

}  // namespace

template <int W, bool ACT>
__global__ __launch_bounds__(kGenThreads) void gen_fwd_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ xh, const bf16 *__restrict__ M,
    bf16 *__restrict__ y, int64_t N, int T, int D, int Dh, int H, int GW, int ncb, float rho) {
  constexpr int GB = kGC / W;  // groups per workgroup
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *At = smem, *Bt = smem + kOffB;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, j = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = blockIdx.x % ncb;
  const int64_t n0 = (int64_t)(blockIdx.x / ncb) * kGT;
  const int col0 = cb * kGC;  // first filter column of the block

  // staging roles: A: 2 vectors (rows ar, ar + 32); B: 8 vectors (rows br + 8i)
  const int ar = tid >> 3, av = tid & 7;
  const int br = tid >> 5, bv = tid & 31;
  const bool bcol_ok = col0 + bv * 8 < GW;  // GW is a multiple of 8
  uint4 ra[2], rb[8];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t n = n0 + ar + 32 * i;
      ra[i] = n < N ? ld16nt(xh + n * Dh + k0 + av * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = bcol_ok ? ld16(M + (int64_t)(k0 + br + 8 * i) * GW + col0 + bv * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4 *>(At + (ar + 32 * i) * kAP + av * 16) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4 *>(Bt + (br + 8 * i) * kBP + bv * 16) = rb[i];
  };

  f32x4g acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = f32x4g{0.f, 0.f, 0.f, 0.f};

  const int nkt = Dh / kGK;
  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load_tile((kt + 1) * kGK);
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      bf16x8g a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)  // rows 16r + j, k = 32 ks + 8q .. +7
        a[r] = __builtin_bit_cast(bf16x8g, *reinterpret_cast<const uint4 *>(
                                               At + (16 * r + j) * kAP + (32 * ks + 8 * q) * 2));
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // k rows 32 ks + 8q .. +7 of column 64 wave + 16 c + j
        const int c0 = 64 * wave + 16 * c;
        const unsigned char *p0 = Bt + (32 * ks + 8 * q + (j >> 2)) * kBP + (c0 + 4 * (j & 3)) * 2;
        const s16x4g lo = tr16g(p0), hi = tr16g(p0 + 4 * kBP);
        const s16x4g v[2] = {lo, hi};
        b[c] = __builtin_bit_cast(bf16x8g, v);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], b[c], acc[r][c], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      store_tile();
      __syncthreads();
    }
  }

  // w tile (bf16) into the B region: token 16r + 4q + e, column 64 wave + 16c + j
  unsigned char *Wt = Bt;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint16_t *>(Wt + (16 * r + 4 * q + e) * kWP +
                                      (64 * wave + 16 * c + j) * 2) =
            __builtin_bit_cast(uint16_t, (__bf16)acc[r][c][e]);
  __syncthreads();

  // convolution: items (channel vector v, token segment s)
  const int ch0 = cb * GB * H;                 // first channel of the block
  const int nv = min(GB * H, D - ch0) / 8;     // channel vectors of the block
  int nseg = 1;  // a power of two, so the segments tile the 64 tokens exactly
  while (2 * nseg * nv <= kGenThreads && 2 * nseg <= kGT) nseg *= 2;
  const int seg = kGT / nseg;
  for (int item = tid; item < nv * nseg; item += kGenThreads) {
    const int v = item % nv, sgi = item / nv;
    const int c = ch0 + v * 8;
    const int gl = (c / H) - cb * GB;          // group inside the block
    const int tl0 = sgi * seg;
    float win[W][8];
    // the window before the segment's first token (same sequence only)
    {
      const int64_t n = n0 + tl0;
      const int t = (int)(n % T);
#pragma unroll
      for (int k = 1; k < W; ++k) {
        if (t - k >= 0 && n < N) {
          unpack<bf16>(ld16(x + (n - k) * D + c), win[k - 1]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) win[k - 1][i] = 0.f;
        }
      }
    }
    for (int tl = tl0; tl < tl0 + seg; ++tl) {
      const int64_t n = n0 + tl;
      if (n >= N) break;
      if (n % T == 0) {  // a sequence starts: nothing before it
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
          for (int i = 0; i < 8; ++i) win[k][i] = 0.f;
      }
#pragma unroll
      for (int k = W - 1; k > 0; --k)
#pragma unroll
        for (int i = 0; i < 8; ++i) win[k][i] = win[k - 1][i];
      unpack<bf16>(ld16nt(x + n * D + c), win[0]);
      float taps[W];
      unpack_row<bf16, W>(ld_row<bf16, W>(reinterpret_cast<const bf16 *>(Wt + tl * kWP) + gl * W),
                          taps);
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k) s = fmaf(taps[k], win[k][i], s);
        if constexpr (ACT) s = silu_f(s);
        o[i] = fmaf(rho, win[0][i], s);
      }
      st16nt(y + n * D + c, pack<bf16>(o));
    }
  }
}

template <int W>
static hipError_t launch_gen(const GenArgs &a) {
  const int64_t N = a.B * a.T;
  if (N == 0) return hipSuccess;
  const int G = (int)(a.D / a.H), GW = G * a.W;
  const int ncb = (GW + kGC - 1) / kGC;
  const int64_t nblocks = (N + kGT - 1) / kGT * ncb;
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  if (a.act)
    hipLaunchKernelGGL((gen_fwd_kernel<W, true>), dim3((unsigned)nblocks), dim3(kGenThreads),
                       kLdsBytes, s, (const bf16 *)a.x, (const bf16 *)a.xh, (const bf16 *)a.M,
                       (bf16 *)a.y, N, (int)a.T, (int)a.D, (int)a.Dh, a.H, GW, ncb, rho);
  else
    hipLaunchKernelGGL((gen_fwd_kernel<W, false>), dim3((unsigned)nblocks), dim3(kGenThreads),
                       kLdsBytes, s, (const bf16 *)a.x, (const bf16 *)a.xh, (const bf16 *)a.M,
                       (bf16 *)a.y, N, (int)a.T, (int)a.D, (int)a.Dh, a.H, GW, ncb, rho);
  return hipGetLastError();
}

hipError_t gen_launch(const GenArgs &a) {
  switch (a.W) {
    case 1: return launch_gen<1>(a);
    case 2: return launch_gen<2>(a);
    case 4: return launch_gen<4>(a);
    case 8: return launch_gen<8>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsc
