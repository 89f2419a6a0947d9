// gen.hip -- head-wise dynamic short convolution with the filters generated on
// chip from a hidden state: w[n, :] = xh[n, :] M, then y as in the head-wise
// forward.  w never reaches device memory.  M arrives transposed, as Mt
// (G*W, Dh) (the weight layout of a linear layer), so that both GEMM operands
// are contiguous along the reduction index Dh.
//
// Operation: gist.science summary "Dynamische Korte Convoluties Verbeteren
// Transformers", Methodologie > Dynamische Korte Convoluties (bullets
// Mechanisme and Parametrisatie: the filter is a learned linear map of the
// hidden state; Parametrisatie 2, head-wise tying); the wispaper.ai blog
// "Dynamic Short Convolutions", Limitations, names merging the convolution into
// the preceding matrix product as the next step for inference.
//
// Mapping: a workgroup of 4 waves owns 128 tokens (flattened b*T + t) and NC
// = 128 filter columns (the tile code also takes 192 and 256), i.e. NC / W
// groups of H channels.  Workgroups are dealt to the 8 XCDs in turn; the
// launch order gives each XCD one group of column blocks over a contiguous
// range of token tiles, so its L2 holds that group's slice of M and each xh
// tile while the group's column blocks use it.
//   * GEMM: the 128 x NC tile of w = xh M accumulates over Dh in K-tiles of
//     32 through a ring of 3 LDS stages.  Tiles (128 xh rows and NC Mt rows of
//     64 bytes) are copied from device memory straight into LDS
//     (global_load_lds_dwordx4), three K-tiles ahead of the one being
//     multiplied, with one barrier per K-tile.  The waves form a 2 x 2 grid of
//     64 x NC/2 sub-tiles computed with 16x16x32 bf16 MFMAs whose A and B
//     fragments are both 16-byte LDS reads, issued one K-tile ahead of their
//     MFMAs.  Rows are XOR-swizzled in 16-byte granules so that these reads
//     are free of bank conflicts; the swizzle is applied on the device-memory
//     side of the copy, since a copy instruction fills 1 KiB of LDS in lane
//     order.
//   * Epilogue: the tile is rounded to bf16 (the precision a stored w would
//     have) into LDS; each thread then owns one 16-byte channel vector and a
//     run of consecutive tokens, keeping the causal window in registers with
//     the next 8 rows of x loaded while the current 8 are used (window slots
//     instead of shifts), and stores y in 16-byte non-temporal writes.  A
//     token tile may span sequences; the window restarts at every sequence
//     start.
// Token rows past the end and filter columns past G*W are read clamped to the
// last valid row / column: they only feed w entries that are never used.
#include "dsc_device.hpp"
#include "gen_launch.hpp"

namespace dsc {

namespace {

typedef __bf16 bf16x8g __attribute__((ext_vector_type(8)));
typedef float f32x4g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGenThreads = 256;
constexpr int kGT = 128;                   // tokens per workgroup
constexpr int kGK = 32;                    // K-tile
constexpr int kStages = 3;                 // LDS ring depth
constexpr int kABytes = kGT * kGK * 2;     // A tile: 128 rows of 64 bytes
constexpr int kUN = 8;                     // x rows per group in the epilogue (a multiple of W)

template <int NC> struct GenTile {
  static_assert(NC == 128 || NC == 192 || NC == 256, "column tile");
  static constexpr int Stage = (kGT + NC) * kGK * 2;   // A rows, then B rows
  static constexpr int WP = NC * 2 + 16;               // w tile row pitch (bytes)
  static constexpr int Lds = kStages * Stage > kGT * WP ? kStages * Stage : kGT * WP;
  static constexpr int NBI = NC / 64;                  // B copies per wave per stage
  static constexpr int NI = 2 + NBI;                   // copies per wave per stage
  static constexpr int CB = NC / 32;                   // 16-column blocks per wave
};

// Granule swizzle of a 64-byte tile row r (4 granules of 8 bf16 along k):
// lane (q, j) reads granule q of row j of a 16-row block at physical granule
// q ^ swz(j).  gfx950's LDS has 64 four-byte banks and serves a 16-byte read
// 16 lanes per pass; measured with a probe, the 16 lanes of a pass are not
// lanes 16p .. 16p+15 but are grouped by lane bit 5 and the parity of lane
// bits 2..4 (possibly with bit 0 or 1: those groupings fit the measurements
// as well).  The plain q ^ (j >> 2) puts two lanes of such a pass on one
// 4-bank window (reads ran at half rate); the permutation 0, 2, 3, 1 of
// j >> 2 leaves every pass on 16 distinct windows under each of these
// groupings and under the consecutive one.
__device__ __forceinline__ int swz(int r) { return (0x78 >> (2 * ((r >> 2) & 3))) & 3; }

// 16 bytes per lane from device memory into LDS at dst + 16 * lane (dst is
// wave-uniform).
__device__ __forceinline__ void copy_lds16(const void *src, unsigned char *dst) {
  __builtin_amdgcn_global_load_lds(
      src, (lds_void *)(__attribute__((address_space(3))) char *)(uintptr_t)dst, 16, 0, 0);
}

// Wait until at most N of this wave's copies are in flight (vmcnt), leaving
// the other counters alone.
template <int N> __device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses but leaves device-memory copies
// in flight (a full __syncthreads would also drain those).
// The wait is also issued as a builtin, which the compiler's own wait
// placement sees: fragments read before the barrier then count as arrived, and
// reads issued after it are waited for only where they are used.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

// ---- GEMM of one 128 x NC tile of w, by four waves of the workgroup -------
// GemmTile holds one wave's part: its copy sources, its LDS read offsets and
// the ring of kStages stages at `stages`.  Wave gw (0..3) computes the
// 64 x NC/2 sub-tile token wm*64 + 16r + 4q + e, column wn*NC/2 + 16c + j
// (wm = gw / 2, wn = gw % 2) with 16x16x32 bf16 MFMAs.
template <int NC> struct GemmTile {
  using Tl = GenTile<NC>;
  unsigned char *stages;
  const bf16 *asrc[2], *bsrc[Tl::NBI];
  int gw, aoff, boff;

  __device__ __forceinline__ GemmTile(unsigned char *st, int gwave, int lane)
      : stages(st), gw(gwave) {
    const int q = lane >> 4, j = lane & 15;
    // fragment row 16 m + j, granule q (k = 8q .. 8q+7); the swizzle depends on j only
    const int foff = j * 64 + 16 * (q ^ swz(j));
    aoff = (gw >> 1) * 64 * 64 + foff;
    boff = kABytes + (gw & 1) * (NC / 2) * 64 + foff;
  }
  // Copy sources of the tile at token n0, column col0.  A copy i of the wave
  // fills tile rows 16 (2 gw + i) .. +15, B copy i rows 16 (gw NBI + i) ..
  // +15; lane l fills granule l & 3 of row l >> 2 with the granule of k that
  // the swizzle puts there.  Rows past N and columns past GW read the last
  // valid one.
  __device__ __forceinline__ void at(const bf16 *__restrict__ xh, const bf16 *__restrict__ Mt,
                                     int64_t n0, int col0, int64_t N, int Dh, int GW, int lane) {
    const int crow = lane >> 2, cgr = 8 * ((lane & 3) ^ swz(crow));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t n = min(n0 + (2 * gw + i) * 16 + crow, N - 1);
      asrc[i] = xh + n * Dh + cgr;
    }
#pragma unroll
    for (int i = 0; i < Tl::NBI; ++i) {
      const int col = min(col0 + (gw * Tl::NBI + i) * 16 + crow, GW - 1);
      bsrc[i] = Mt + (int64_t)col * Dh + cgr;
    }
  }
  // K-tile kt (32 values of k) into ring stage st
  __device__ __forceinline__ void issue(int kt, int st) const {
    unsigned char *P = stages + st * Tl::Stage;
    const int k0 = kt * kGK;
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_lds16(asrc[i] + k0, P + 1024 * (2 * gw + i));
#pragma unroll
    for (int i = 0; i < Tl::NBI; ++i)
      copy_lds16(bsrc[i] + k0, P + kABytes + 1024 * (gw * Tl::NBI + i));
  }
  __device__ __forceinline__ void rd(int kt, bf16x8g (&a)[4], bf16x8g (&b)[Tl::CB]) const {
    const unsigned char *P = stages + (kt % kStages) * Tl::Stage;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      a[r] = __builtin_bit_cast(bf16x8g, *reinterpret_cast<const uint4 *>(P + aoff + 1024 * r));
#pragma unroll
    for (int c = 0; c < Tl::CB; ++c)
      b[c] = __builtin_bit_cast(bf16x8g, *reinterpret_cast<const uint4 *>(P + boff + 1024 * c));
  }
  static __device__ __forceinline__ void mm(const bf16x8g (&a)[4], const bf16x8g (&b)[Tl::CB],
                                            f32x4g (&acc)[4][Tl::CB]) {
#pragma unroll
    for (int c = 0; c < Tl::CB; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], b[c], acc[r][c], 0, 0, 0);
  }
  static __device__ __forceinline__ void zero(f32x4g (&acc)[4][Tl::CB]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < Tl::CB; ++c) acc[r][c] = f32x4g{0.f, 0.f, 0.f, 0.f};
  }
};

// The whole K loop of one tile by waves 0..3, nkt = Dh / 32 K-tiles (even):
// copies run up to three K-tiles ahead through the ring, one lds_barrier per
// K-tile, and each K-tile's fragments are read from LDS one K-tile ahead,
// while the MFMAs of the previous one run, so the LDS latency hides behind
// them.  Every wave of the workgroup must call it (the barriers).
template <int NC>
__device__ __forceinline__ void gen_gemm(unsigned char *stages, const bf16 *__restrict__ xh,
                                         const bf16 *__restrict__ Mt, int64_t n0, int col0,
                                         int64_t N, int Dh, int GW, int wave, int lane,
                                         f32x4g (&acc)[4][GenTile<NC>::CB]) {
  using Tl = GenTile<NC>;
  GemmTile<NC> g(stages, wave, lane);
  g.at(xh, Mt, n0, col0, N, Dh, GW, lane);
  GemmTile<NC>::zero(acc);
  const int nkt = Dh / kGK;  // even (Dh is a multiple of 64)
  g.issue(0, 0);
  g.issue(1, 1);
  if (nkt > 2) {
    g.issue(2, 2);
    wait_copies<2 * Tl::NI>();
  } else {
    wait_copies<Tl::NI>();
  }
  lds_barrier();  // tile 0 is in LDS for every wave
  bf16x8g a0[4], b0[Tl::CB], a1[4], b1[Tl::CB];
  g.rd(0, a0, b0);
  // step kt < nkt - 2: the fragments of tile kt are in (ac, bc); those of
  // kt + 1 go to (an, bn).  The last two steps are peeled so that no branch
  // skips a barrier inside the loop (a path without one would make the
  // compiler wait for every LDS read before the MFMAs).
  auto step = [&](int kt, bf16x8g(&ac)[4], bf16x8g(&bc)[Tl::CB], bf16x8g(&an)[4],
                  bf16x8g(&bn)[Tl::CB]) {
    wait_copies<Tl::NI>();  // tile kt + 1 landed; kt + 2 may be in flight
    // tile kt + 1 is in LDS for every wave, and every wave holds its
    // fragments of tile kt, whose stage the next copy overwrites
    lds_barrier();
    if (kt + 3 < nkt) g.issue(kt + 3, kt % kStages);
    g.rd(kt + 1, an, bn);
    GemmTile<NC>::mm(ac, bc, acc);
  };
  for (int kt = 0; kt < nkt - 2; kt += 2) {
    step(kt, a0, b0, a1, b1);
    step(kt + 1, a1, b1, a0, b0);
  }
  wait_copies<0>();
  lds_barrier();
  g.rd(nkt - 1, a1, b1);
  GemmTile<NC>::mm(a0, b0, acc);
  GemmTile<NC>::mm(a1, b1, acc);
}

// The accumulators of gen_gemm, rounded to bf16, into a w tile of 128 rows of
// pitch WP bytes (row = token of the tile, column = filter column g*W + k).
template <int NC>
__device__ __forceinline__ void gen_store_w(unsigned char *wt, int wave, int lane,
                                            const f32x4g (&acc)[4][GenTile<NC>::CB]) {
  using Tl = GenTile<NC>;
  const int q = lane >> 4, j = lane & 15, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < Tl::CB; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint16_t *>(wt + (wm * 64 + 16 * r + 4 * q + e) * Tl::WP +
                                      (wn * (NC / 2) + 16 * c + j) * 2) =
            __builtin_bit_cast(uint16_t, (__bf16)acc[r][c][e]);
}

// Tile b of the launch order -> column block cb, token tile tt.  With ngrp >
// 0 (see gen_groups), tiles go to the 8 XCDs in turn (b & 7 is the XCD of a
// workgroup dealt in launch order): XCD x runs column blocks of group
// x / (8 / ngrp) for a contiguous range of token tiles, the column blocks of
// one token tile one after another, so its L2 keeps that group's M slice and
// each xh tile while they are used.
__device__ __forceinline__ void gen_tile_at(int b, int ncb, int ntt, int ngrp, int &cb, int &tt) {
  if (ngrp > 0) {
    const int xcd = b & 7, slot = b >> 3;
    const int xpg = 8 / ngrp, cpg = ncb / ngrp;
    cb = (xcd / xpg) * cpg + slot % cpg;
    tt = (xcd % xpg) * (ntt / xpg) + slot / cpg;
  } else {
    cb = b % ncb;
    tt = b / ncb;
  }
}

// Segments of a column block's convolution: nv vectors of 8 channels, each
// token run `seg` = 128 / nseg long, nseg a power of two with nseg * nv <=
// threads and seg >= minseg.
__host__ __device__ __forceinline__ int gen_nseg(int nv, int threads, int minseg) {
  int nseg = 1;
  while (2 * nseg * nv <= threads && kGT / (2 * nseg) >= minseg) nseg *= 2;
  return nseg;
}

// ---------------------------------------------------------------------------
// The kernel: GEMM of the tile, then its convolution, by all 4 waves.
// ---------------------------------------------------------------------------
template <int W, int NC, bool ACT>
__global__ __launch_bounds__(kGenThreads, 2) void gen_fwd_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ xh, const bf16 *__restrict__ Mt,
    bf16 *__restrict__ y, int64_t N, int T, int D, int Dh, int H, int GW, int ncb, int ntt,
    int ngrp, float rho) {
  using Tl = GenTile<NC>;
  static_assert(kUN % W == 0, "window slots repeat every W tokens of a group");
  constexpr int GB = NC / W;  // groups per workgroup
  __shared__ __align__(16) unsigned char smem[Tl::Lds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int cb, tt;
  gen_tile_at((int)blockIdx.x, ncb, ntt, ngrp, cb, tt);
  const int64_t n0 = (int64_t)tt * kGT;

  f32x4g acc[4][Tl::CB];
  gen_gemm<NC>(smem, xh, Mt, n0, cb * NC, N, Dh, GW, wave, lane, acc);
  lds_barrier();  // every wave is done with the last stage
  gen_store_w<NC>(smem, wave, lane, acc);
  __syncthreads();

  // convolution: items (channel vector v, token segment)
  const int ch0 = cb * GB * H;              // first channel of the block
  const int nv = min(GB * H, D - ch0) / 8;  // channel vectors of the block
  const int seg = kGT / gen_nseg(nv, kGenThreads, kUN);
  for (int item = tid; item < nv * (kGT / seg); item += kGenThreads) {
    const int v = item % nv, sgi = item / nv;
    const int c = ch0 + v * 8;
    const int gl = c / H - cb * GB;  // group inside the block
    const int tl0 = sgi * seg;
    if (n0 + tl0 >= N) continue;
    int t = (int)((n0 + tl0) % T);
    // rows of the segment; loads past its last row repeat that row (cache
    // hits), so every load is unconditional and a group of kUN rows can be in
    // flight while the previous one is used
    const int64_t nlast = min(N, n0 + tl0 + seg) - 1;
    auto xrow = [&](int64_t n) { return ld16nt(x + min(n, nlast) * D + c); };
    // window slots: slot u % W holds the token at offset u of a group (kUN is
    // a multiple of W), the slots before the first group hold the W-1 tokens
    // before the segment (zero before a sequence start)
    float win[W][8];
#pragma unroll
    for (int k = 1; k < W; ++k) {
      const int sl = (W - k) % W;
      if (t - k >= 0) {
        unpack<bf16>(ld16(x + (n0 + tl0 - k) * D + c), win[sl]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) win[sl][i] = 0.f;
      }
    }
    uint4 xc[kUN];
#pragma unroll
    for (int u = 0; u < kUN; ++u) xc[u] = xrow(n0 + tl0 + u);
    for (int tl = tl0; tl < tl0 + seg; tl += kUN) {
      uint4 xn[kUN];
#pragma unroll
      for (int u = 0; u < kUN; ++u) xn[u] = xrow(n0 + tl + kUN + u);
#pragma unroll
      for (int u = 0; u < kUN; ++u) {
        const int64_t n = n0 + tl + u;
        if (n <= nlast) {
          const int sl = u % W;
          if (t == 0) {  // a sequence starts: nothing before it
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
              for (int i = 0; i < 8; ++i) win[k][i] = 0.f;
          }
          unpack<bf16>(xc[u], win[sl]);
          float taps[W];
          unpack_row<bf16, W>(
              ld_row<bf16, W>(reinterpret_cast<const bf16 *>(smem + (tl + u) * Tl::WP) + gl * W),
              taps);
          float o[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < W; ++k) s = fmaf(taps[k], win[(sl - k + W) % W][i], s);
            if constexpr (ACT) s = silu_f(s);
            o[i] = fmaf(rho, win[sl][i], s);
          }
          st16nt(y + n * D + c, pack<bf16>(o));
          if (++t == T) t = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kUN; ++u) xc[u] = xn[u];
    }
  }
}

namespace {

// Column groups for the XCD-aware order of gen_fwd_kernel: the fewest groups
// g in {2, 4, 8} such that g divides the column-block count, 8 / g divides
// the token-tile count and a group's M slice (ncb / g blocks of NC x Dh bf16)
// takes at most 3 MiB of an XCD's 4 MiB L2; 0 (plain order) when none fits.
// At B=8 T=2048 D=6144 Dh=2048 W=4 H=16 (12 column blocks, 3 MiB slices at
// g = 2) this order measured 178 us against 190 us for the plain one, with
// L2 misses down from 808 MB to 457 MB per call; g = 4 measured 182 us.
int gen_groups(int64_t ntt, int ncb, int nc, int64_t Dh) {
  for (int g : {2, 4, 8}) {
    if (ncb % g || ntt % (8 / g)) continue;
    if ((int64_t)(ncb / g) * nc * Dh * 2 <= (3 << 20)) return g;
  }
  return 0;
}

template <int W, int NC>
hipError_t launch_gen_nc(const GenArgs &a, int64_t N, int GW) {
  const int ncb = (GW + NC - 1) / NC;
  const int64_t ntt = (N + kGT - 1) / kGT;
  const int64_t nblocks = ntt * ncb;
  if (nblocks > INT32_MAX) return hipErrorInvalidValue;
  const int ngrp = gen_groups(ntt, ncb, NC, a.Dh);
  const float rho = a.residual ? 1.f : 0.f;
  hipStream_t s = (hipStream_t)a.stream;
  if (a.act)
    hipLaunchKernelGGL((gen_fwd_kernel<W, NC, true>), dim3((unsigned)nblocks), dim3(kGenThreads),
                       0, s, (const bf16 *)a.x, (const bf16 *)a.xh, (const bf16 *)a.Mt,
                       (bf16 *)a.y, N, (int)a.T, (int)a.D, (int)a.Dh, a.H, GW, ncb, (int)ntt,
                       ngrp, rho);
  else
    hipLaunchKernelGGL((gen_fwd_kernel<W, NC, false>), dim3((unsigned)nblocks), dim3(kGenThreads),
                       0, s, (const bf16 *)a.x, (const bf16 *)a.xh, (const bf16 *)a.Mt,
                       (bf16 *)a.y, N, (int)a.T, (int)a.D, (int)a.Dh, a.H, GW, ncb, (int)ntt,
                       ngrp, rho);
  return hipGetLastError();
}

// Column tile 128: three workgroups fit a CU (48 KiB of LDS, about 110
// VGPRs), and on MI355X at B=8 T=2048 D=6144 Dh=2048 W=4 H=16 it beats the
// wider tiles (194 us against 219 us for 192 and 218 us for 256 columns),
// whose GEMM alone is faster (113 us for 256 against 130 us for 128) but
// which keep two workgroups per CU, so fewer GEMM and convolution phases of
// different workgroups overlap.
template <int W>
hipError_t launch_gen(const GenArgs &a) {
  const int64_t N = a.B * a.T;
  if (N == 0) return hipSuccess;
  return launch_gen_nc<W, 128>(a, N, (int)(a.D / a.H) * a.W);
}

}  // namespace

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
