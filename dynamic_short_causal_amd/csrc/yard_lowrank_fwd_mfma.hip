// yard_lowrank_fwd_mfma.hip -- a measurement yardstick, not part of libdsc.so:
// the matrix-core low-rank forward (lr_fwd_kernel) for bf16 filters tied over
// H = 8 channels, the case libdsc.so serves with the vector-ALU kernel
// (lowrank_fwd_valu.hpp).  libdsc_yard.so is loaded only by the benchmark's
// --tied8-forward mode, which times both kernels on the same inputs so that
// the choice between them rests on a measurement that can be repeated.
#include "lowrank_launch.hpp"

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

}  // extern "C"
