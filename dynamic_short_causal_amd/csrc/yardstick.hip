// yardstick.hip -- measurement yardsticks, not part of libdsc.so.  They are
// the other side of choices libdsc.so makes between kernels, built into
// libdsc_yard.so and loaded only by the benchmark's --tied8-forward and
// --tied8-backward modes, which time both sides on the same inputs so the
// choices rest on measurements that can be repeated:
//   * dsc_yard_lowrank_fwd_mfma: the matrix-core low-rank forward
//     (lr_fwd_kernel) for bf16 filters tied over H = 8 channels, the case
//     libdsc.so serves with the vector-ALU forward (lowrank_fwd_valu.hpp);
//   * dsc_yard_lowrank_bwd_valu: the vector-ALU low-rank backward
//     (lowrank_bwd_valu.hpp) for the same case, which libdsc.so serves with
//     the matrix-core backward (lr_bwd_kernel).
#include "lowrank_launch.hpp"
#include "lowrank_bwd_valu.hpp"

extern "C" {

// Same operation and layouts as dsc_lowrank_fwd (bf16 only, W = 4, H = 8,
// R <= 16, no packed rows): x, y (B, T, D); z (B, T, R); U (R, (D/8)*4), all
// device pointers; stream is a hipStream_t.  Returns 0, -1 for arguments
// outside that case, else the HIP error code.
int dsc_yard_lowrank_fwd_mfma(const void *x, const void *z, const void *U, void *y, int64_t B,
                              int64_t T, int64_t D, int R, int residual, int act, void *stream) {
  if (!x || !z || !U || !y || B < 0 || T < 0 || D <= 0 || D % 8 || R < 1 || R > 16) return -1;
  dsc::LrArgs a{};
  a.x = x; a.z = z; a.U = U; a.y = y;
  a.B = B; a.T = T; a.D = D; a.W = 4; a.H = 8; a.R = R;
  a.bf16 = true; a.residual = residual != 0; a.act = act != 0; a.bwd = false;
  a.stream = stream;
  const hipError_t e = act ? dsc::launch_lr_fwd_mfma<dsc::bf16, 4, 1, true, false, 1>(a)
                           : dsc::launch_lr_fwd_mfma<dsc::bf16, 4, 1, false, false, 1>(a);
  return e == hipSuccess ? 0 : (int)e;
}

// Workspace bytes of dsc_yard_lowrank_bwd_valu (fp32 partials of dz and dU).
size_t dsc_yard_lowrank_bwd_valu_workspace(int64_t B, int64_t T, int64_t D) {
  if (B < 0 || T < 0 || D <= 0 || D % 8) return 0;
  return dsc::lr_bwd_valu_plan(B, T, D, 4).bytes;
}

// Same operation and layouts as dsc_lowrank_bwd (bf16, W = 4, H = 8, even
// R <= 16, no packed rows): x, dy, dx (B, T, D); z, dz (B, T, R); U, dU
// (R, (D/8)*4); ws at least dsc_yard_lowrank_bwd_valu_workspace bytes.
// Device pointers; stream is a hipStream_t.  Returns 0, -1 for arguments
// outside that case, else the HIP error code.
int dsc_yard_lowrank_bwd_valu(const void *x, const void *z, const void *U, const void *dy, void *dx,
                              void *dz, void *dU, void *ws, int64_t B, int64_t T, int64_t D, int R,
                              int residual, int act, void *stream) {
  if (!x || !z || !U || !dy || !dx || !dz || !dU || !ws || B < 0 || T < 0 || D <= 0 || D % 8)
    return -1;
  if (!dsc::lr_bwd_uses_valu(true, D, 4, 8, R, false)) return -1;
  dsc::LrArgs a{};
  a.x = x; a.z = z; a.U = U; a.dy = dy; a.dx = dx; a.dz = dz; a.dU = dU; a.ws = ws;
  a.B = B; a.T = T; a.D = D; a.W = 4; a.H = 8; a.R = R;
  a.bf16 = true; a.residual = residual != 0; a.act = act != 0; a.bwd = true;
  a.stream = stream;
  const dsc::LbPlan p = dsc::lr_bwd_valu_plan(B, T, D, 4);
  float *dzp = (float *)ws;
  float *dUp = (float *)((char *)ws + p.dz_part);
  hipError_t e = act ? dsc::launch_lr_bwd_valu<4, true>(a, dzp, dUp)
                     : dsc::launch_lr_bwd_valu<4, false>(a, dzp, dUp);
  if (e == hipSuccess) {
    dsc::LrBwdPlan rp{};
    rp.rpad = 16;
    rp.ncb = p.nvb;
    rp.nchunk = p.nchunk;
    e = dsc::launch_lr_reduce<dsc::bf16>(a, rp, dzp, dUp);
  }
  return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
