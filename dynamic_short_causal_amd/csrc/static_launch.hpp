// static_launch.hpp -- host-side arguments and tiling of the static-filter
// kernels in static.hip, shared by the C ABI (checks, workspace query) and the
// launchers so the two always agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsc {

// x, y, dy, dx (B, T, D); w, dw (G, W) with G = D / H.
struct StArgs {
  const void *x, *w, *dy;
  void *y, *dx, *dw, *ws;
  int64_t B, T, D;
  int W, H;
  bool bf16, residual, act, bwd;
  void *stream;
};

// The forward gives each lane a chunk of kStFwdChunk tokens.  The backward
// gives each wave a chunk of kStChunk tokens and each workgroup kStWaves
// consecutive chunks of the same channels; one fp32 partial row of dw (G * W
// values) per (sequence, chunk group) goes to the workspace.  Measured at
// B=8, T=2048, D=6144, W=4 (bf16): backward chunks of 128 tokens run in
// 127 us against 139 us for 64 (fewer halo re-reads and partial rows); the
// forward is flat between 32 and 128 and slower at 256.
constexpr int kStFwdChunk = 64;
constexpr int kStChunk = 128;
constexpr int kStWaves = 4;

struct StPlan {
  int tc, nchunk, ncg;
  int64_t parts;  // B * ncg
  size_t bytes;   // parts * G * W * 4
};

inline StPlan st_plan(int64_t B, int64_t T, int64_t D, int W, int H) {
  StPlan p{};
  p.tc = T < kStChunk ? (int)(T > 0 ? T : 1) : kStChunk;
  p.nchunk = (int)((T + p.tc - 1) / p.tc);
  p.ncg = (p.nchunk + kStWaves - 1) / kStWaves;
  p.parts = B * p.ncg;
  p.bytes = (size_t)p.parts * (size_t)(D / H) * (size_t)W * sizeof(float);
  return p;
}

hipError_t static_launch(const StArgs &a);

}  // namespace dsc
