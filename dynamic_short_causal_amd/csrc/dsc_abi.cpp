// dsc_abi.cpp -- the C ABI declared in include/dsc.h: host-side argument
// checks, then dispatch to the gfx950 kernel launchers.  No allocation, no
// synchronisation, no state kept between calls.
#include "../../include/dsc.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "dsc_launch.hpp"
#include "decode_launch.hpp"
#include "static_launch.hpp"
#include "gen_launch.hpp"

namespace {

thread_local char g_err[512] = "";

dsc_status fail(dsc_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

dsc_status ok() {
  g_err[0] = '\0';
  return DSC_OK;
}

struct Span {
  const char *name;
  uintptr_t lo, hi;  // [lo, hi) bytes; empty when lo == hi
  bool output;
};

bool overlap(const Span &a, const Span &b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Activation tensors above 2^38 elements exceed one GPU's memory by far; the
// bound also keeps every launch grid below 2^31 workgroups.
const int64_t kMaxElems = (int64_t)1 << 38;

// Common shape / dtype / flag checks.  On success sets *V.
dsc_status check_common(int64_t B, int64_t T, int64_t D, int W, int H, dsc_dtype dtype,
                        unsigned flags, int *V) {
  if (dtype != DSC_F32 && dtype != DSC_BF16)
    return fail(DSC_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (flags & ~(DSC_RESIDUAL | DSC_ACT_SILU))
    return fail(DSC_ERR_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (B < 0 || T < 0) return fail(DSC_ERR_INVALID_ARG, "B=%lld and T=%lld must be >= 0",
                                  (long long)B, (long long)T);
  if (D < 1) return fail(DSC_ERR_INVALID_ARG, "D=%lld must be >= 1", (long long)D);
  if (B > INT32_MAX || T > INT32_MAX || D > INT32_MAX)
    return fail(DSC_ERR_INVALID_ARG, "B, T and D must each be below 2^31");
  if (B > 0 && T > 0 && (B * T > kMaxElems / D))
    return fail(DSC_ERR_INVALID_ARG, "B*T*D exceeds 2^38 elements");
  if (W < 1 || W > 8) return fail(DSC_ERR_UNSUPPORTED, "W=%d outside 1..8", W);
  if (H < 1) return fail(DSC_ERR_INVALID_ARG, "H=%d must be >= 1", H);
  if (D % H) return fail(DSC_ERR_INVALID_ARG, "D=%lld is not a multiple of H=%d",
                         (long long)D, H);
  *V = dtype == DSC_BF16 ? 8 : 4;
  if (D % *V)
    return fail(DSC_ERR_INVALID_ARG, "D=%lld is not a multiple of the %d-element vector",
                (long long)D, *V);
  return DSC_OK;
}

dsc_status check_ptrs(const Span *s, int n) {
  for (int i = 0; i < n; ++i) {
    if (s[i].lo == s[i].hi) continue;  // empty tensor: pointer not used
    if (s[i].lo == 0) return fail(DSC_ERR_INVALID_ARG, "%s is NULL", s[i].name);
    if (s[i].lo % 16) return fail(DSC_ERR_INVALID_ARG, "%s is not 16-byte aligned", s[i].name);
  }
  for (int i = 0; i < n; ++i) {
    if (!s[i].output) continue;
    for (int j = 0; j < n; ++j) {
      if (j == i || (s[j].output && j < i)) continue;
      if (overlap(s[i], s[j]))
        return fail(DSC_ERR_INVALID_ARG, "output %s overlaps %s", s[i].name, s[j].name);
    }
  }
  return DSC_OK;
}

Span span(const char *name, const void *p, int64_t elems, int esize, bool out) {
  uintptr_t lo = (uintptr_t)p;
  return Span{name, lo, lo + (uintptr_t)(elems * esize), out};
}

// H divides the vector width (whole groups in one vector), or a group spans
// L = H / V whole vectors, at most one wave's 64 lanes
bool headwise_h_ok(int H, int V) {
  if (V % H == 0) return true;
  return H % V == 0 && H / V <= 64;
}

dsc_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(DSC_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

// Partial-sum buffer of dsc_lowrank_bwd_noalloc, owned by the library: every
// GPU the library runs on holds its own copy (a zero-filled .bss segment of
// the code object, 128 MiB) until the process ends.  In host code `scratch`
// names a host-side stand-in, never device memory: kernels get the device
// address looked up below.
constexpr size_t kScratchBytes = (size_t)DSC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device ordinal

// Device address of `scratch` on the current device, looked up with that
// device current on the first call there and kept.
dsc_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSC_ERR_HIP, "device ordinal %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || ((uintptr_t)p % 256) != 0)
      return fail(DSC_ERR_HIP, "scratch buffer of device %d at %p", dev, p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSC_OK;
}

}  // namespace

extern "C" {

int dsc_version(void) { return 10000; }

const char *dsc_status_string(dsc_status s) {
  switch (s) {
    case DSC_OK: return "DSC_OK";
    case DSC_ERR_INVALID_ARG: return "DSC_ERR_INVALID_ARG";
    case DSC_ERR_UNSUPPORTED: return "DSC_ERR_UNSUPPORTED";
    case DSC_ERR_WORKSPACE: return "DSC_ERR_WORKSPACE";
    case DSC_ERR_HIP: return "DSC_ERR_HIP";
  }
  return "DSC_ERR_UNKNOWN";
}

const char *dsc_last_error(void) { return g_err; }

static dsc_status headwise_common(const void *x, const void *w, const void *dy,
                                  const int32_t *pos, bool varlen, void *y, void *dx, void *dw,
                                  int64_t B, int64_t T, int64_t D, int W, int H,
                                  dsc_dtype dtype, unsigned flags, void *stream, bool bwd) {
  int V = 0;
  dsc_status st = check_common(B, T, D, W, H, dtype, flags, &V);
  if (st != DSC_OK) return st;
  if (!headwise_h_ok(H, V))
    return fail(DSC_ERR_UNSUPPORTED,
                "H=%d: head-wise needs H | %d or H = %d * m with m <= 64", H, V, V);
  const int es = dtype == DSC_BF16 ? 2 : 4;
  const int64_t n_act = B * T * D, n_w = B * T * (D / H) * W;
  const Span sp = span("pos", pos, varlen ? B * T : 0, 4, false);
  if (!bwd) {
    Span s[4] = {span("x", x, n_act, es, false), span("w", w, n_w, es, false),
                 span("y", y, n_act, es, true), sp};
    if ((st = check_ptrs(s, 4)) != DSC_OK) return st;
  } else {
    Span s[6] = {span("x", x, n_act, es, false), span("w", w, n_w, es, false),
                 span("dy", dy, n_act, es, false), span("dx", dx, n_act, es, true),
                 span("dw", dw, n_w, es, true), sp};
    if ((st = check_ptrs(s, 6)) != DSC_OK) return st;
  }
  dsc::HwArgs a{};
  a.x = x; a.w = w; a.dy = dy; a.y = y; a.dx = dx; a.dw = dw;
  a.pos = varlen ? pos : nullptr;
  a.B = B; a.T = T; a.D = D; a.W = W; a.H = H;
  a.bf16 = dtype == DSC_BF16;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.bwd = bwd;
  a.stream = stream;
  return hip_status(dsc::headwise_launch(a));
}

dsc_status dsc_headwise_fwd(const void *x, const void *w, void *y, int64_t B, int64_t T,
                            int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                            void *stream) {
  return headwise_common(x, w, nullptr, nullptr, false, y, nullptr, nullptr, B, T, D, W, H,
                         dtype, flags, stream, false);
}

dsc_status dsc_headwise_bwd(const void *x, const void *w, const void *dy, void *dx, void *dw,
                            int64_t B, int64_t T, int64_t D, int W, int H, dsc_dtype dtype,
                            unsigned flags, void *stream) {
  return headwise_common(x, w, dy, nullptr, false, nullptr, dx, dw, B, T, D, W, H, dtype, flags,
                         stream, true);
}

dsc_status dsc_headwise_fwd_varlen(const void *x, const void *w, const int32_t *pos, void *y,
                                   int64_t B, int64_t T, int64_t D, int W, int H,
                                   dsc_dtype dtype, unsigned flags, void *stream) {
  return headwise_common(x, w, nullptr, pos, true, y, nullptr, nullptr, B, T, D, W, H, dtype,
                         flags, stream, false);
}

dsc_status dsc_headwise_bwd_varlen(const void *x, const void *w, const int32_t *pos,
                                   const void *dy, void *dx, void *dw, int64_t B, int64_t T,
                                   int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                                   void *stream) {
  return headwise_common(x, w, dy, pos, true, nullptr, dx, dw, B, T, D, W, H, dtype, flags,
                         stream, true);
}

static dsc_status lowrank_check(int64_t B, int64_t T, int64_t D, int W, int H, int R,
                                dsc_dtype dtype, unsigned flags, int *V) {
  dsc_status st = check_common(B, T, D, W, H, dtype, flags, V);
  if (st != DSC_OK) return st;
  if (*V % H && H % *V)
    return fail(DSC_ERR_UNSUPPORTED, "H=%d: low-rank needs H to divide %d or be a multiple of it",
                H, *V);
  if (R < 1 || R > 64) return fail(DSC_ERR_UNSUPPORTED, "R=%d outside 1..64", R);
  return DSC_OK;
}

static dsc_status lowrank_fwd_common(const void *x, const void *z, const void *U,
                                     const int32_t *pos, bool varlen, void *y, int64_t B,
                                     int64_t T, int64_t D, int W, int H, int R, dsc_dtype dtype,
                                     unsigned flags, void *stream) {
  int V = 0;
  dsc_status st = lowrank_check(B, T, D, W, H, R, dtype, flags, &V);
  if (st != DSC_OK) return st;
  const int es = dtype == DSC_BF16 ? 2 : 4;
  const int64_t n_act = B * T * D;
  Span s[5] = {span("x", x, n_act, es, false), span("z", z, B * T * R, es, false),
               span("U", U, (int64_t)R * (D / H) * W, es, false),
               span("y", y, n_act, es, true), span("pos", pos, varlen ? B * T : 0, 4, false)};
  if ((st = check_ptrs(s, 5)) != DSC_OK) return st;
  dsc::LrArgs a{};
  a.x = x; a.z = z; a.U = U; a.y = y;
  a.pos = varlen ? pos : nullptr;
  a.B = B; a.T = T; a.D = D; a.W = W; a.H = H; a.R = R;
  a.bf16 = dtype == DSC_BF16;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.bwd = false;
  a.stream = stream;
  return hip_status(dsc::lowrank_launch(a));
}

dsc_status dsc_lowrank_fwd(const void *x, const void *z, const void *U, void *y, int64_t B,
                           int64_t T, int64_t D, int W, int H, int R, dsc_dtype dtype,
                           unsigned flags, void *stream) {
  return lowrank_fwd_common(x, z, U, nullptr, false, y, B, T, D, W, H, R, dtype, flags, stream);
}

dsc_status dsc_lowrank_fwd_varlen(const void *x, const void *z, const void *U,
                                  const int32_t *pos, void *y, int64_t B, int64_t T, int64_t D,
                                  int W, int H, int R, dsc_dtype dtype, unsigned flags,
                                  void *stream) {
  return lowrank_fwd_common(x, z, U, pos, true, y, B, T, D, W, H, R, dtype, flags, stream);
}

size_t dsc_lowrank_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W, int H, int R,
                                       dsc_dtype dtype) {
  int V = 0;
  if (lowrank_check(B, T, D, W, H, R, dtype, 0, &V) != DSC_OK) return 0;
  return dsc::lr_bwd_workspace(B, T, D, W, H, R, dtype == DSC_BF16);
}

// lib_ws: the partial sums go to the library-owned buffer (dsc_lowrank_bwd_noalloc)
// instead of the caller's workspace; its device address is looked up only
// after every host-side check has passed.
static dsc_status lowrank_bwd_common(const void *x, const void *z, const void *U,
                                     const int32_t *pos, bool varlen, const void *dy, void *dx,
                                     void *dz, void *dU, void *workspace,
                                     size_t workspace_bytes, int64_t B, int64_t T, int64_t D,
                                     int W, int H, int R, dsc_dtype dtype, unsigned flags,
                                     void *stream, bool lib_ws = false) {
  int V = 0;
  dsc_status st = lowrank_check(B, T, D, W, H, R, dtype, flags, &V);
  if (st != DSC_OK) return st;
  const int es = dtype == DSC_BF16 ? 2 : 4;
  // the backward addresses 16-row slabs of x, dy and dx through 32-bit buffer
  // offsets, with 2^31 marking a channel past D
  if (16 * D * es >= ((int64_t)1 << 31))
    return fail(DSC_ERR_UNSUPPORTED, "low-rank backward: 16 rows of D=%lld exceed 2^31 bytes",
                (long long)D);
  const int64_t n_act = B * T * D, n_z = B * T * R, n_U = (int64_t)R * (D / H) * W;
  const size_t need = dsc::lr_bwd_workspace(B, T, D, W, H, R, dtype == DSC_BF16);
  Span s[9] = {span("x", x, n_act, es, false),   span("z", z, n_z, es, false),
               span("U", U, n_U, es, false),     span("dy", dy, n_act, es, false),
               span("dx", dx, n_act, es, true),  span("dz", dz, n_z, es, true),
               span("dU", dU, n_U, es, true),
               span("workspace", lib_ws ? nullptr : workspace, lib_ws ? 0 : (int64_t)need, 1,
                    true),
               span("pos", pos, varlen ? B * T : 0, 4, false)};
  if (lib_ws) {
    if (need > kScratchBytes)
      return fail(DSC_ERR_WORKSPACE,
                  "this shape needs %zu bytes of partial sums, above the %zu-byte library buffer",
                  need, kScratchBytes);
  } else {
    if (need > 0 && workspace_bytes < need)
      return fail(DSC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed",
                  workspace_bytes, need);
    if (need > 0 && workspace == nullptr)
      return fail(DSC_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  }
  if ((st = check_ptrs(s, 9)) != DSC_OK) return st;
  if (lib_ws && need > 0 && (st = scratch_of_current_device(&workspace)) != DSC_OK) return st;
  dsc::LrArgs a{};
  a.x = x; a.z = z; a.U = U; a.dy = dy; a.dx = dx; a.dz = dz; a.dU = dU; a.ws = workspace;
  a.pos = varlen ? pos : nullptr;
  a.B = B; a.T = T; a.D = D; a.W = W; a.H = H; a.R = R;
  a.bf16 = dtype == DSC_BF16;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.bwd = true;
  a.stream = stream;
  return hip_status(dsc::lowrank_launch(a));
}

dsc_status dsc_lowrank_bwd(const void *x, const void *z, const void *U, const void *dy,
                           void *dx, void *dz, void *dU, void *workspace,
                           size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int W,
                           int H, int R, dsc_dtype dtype, unsigned flags, void *stream) {
  return lowrank_bwd_common(x, z, U, nullptr, false, dy, dx, dz, dU, workspace,
                            workspace_bytes, B, T, D, W, H, R, dtype, flags, stream);
}

dsc_status dsc_lowrank_bwd_varlen(const void *x, const void *z, const void *U,
                                  const int32_t *pos, const void *dy, void *dx, void *dz,
                                  void *dU, void *workspace, size_t workspace_bytes, int64_t B,
                                  int64_t T, int64_t D, int W, int H, int R, dsc_dtype dtype,
                                  unsigned flags, void *stream) {
  return lowrank_bwd_common(x, z, U, pos, true, dy, dx, dz, dU, workspace, workspace_bytes, B,
                            T, D, W, H, R, dtype, flags, stream);
}

dsc_status dsc_lowrank_bwd_noalloc(const void *x, const void *z, const void *U, const void *dy,
                                   void *dx, void *dz, void *dU, int64_t B, int64_t T, int64_t D,
                                   int W, int H, int R, dsc_dtype dtype, unsigned flags,
                                   void *stream) {
  return lowrank_bwd_common(x, z, U, nullptr, false, dy, dx, dz, dU, nullptr, 0, B, T, D, W, H,
                            R, dtype, flags, stream, true);
}

static dsc_status decode_common(const void *x, const void *w, const void *z, const void *U,
                                void *state, void *y, int64_t B, int64_t D, int W, int H,
                                int R, dsc_dtype dtype, unsigned flags, void *stream,
                                bool lowrank) {
  int V = 0;
  dsc_status st = lowrank ? lowrank_check(B, 1, D, W, H, R, dtype, flags, &V)
                          : check_common(B, 1, D, W, H, dtype, flags, &V);
  if (st != DSC_OK) return st;
  if (!lowrank && !headwise_h_ok(H, V))
    return fail(DSC_ERR_UNSUPPORTED,
                "H=%d: head-wise needs H | %d or H = %d * m with m <= 64", H, V, V);
  const int es = dtype == DSC_BF16 ? 2 : 4;
  const int64_t G = D / H;
  Span s[5] = {span("x", x, B * D, es, false),
               lowrank ? span("z", z, B * R, es, false) : span("w", w, B * G * W, es, false),
               span("U", lowrank ? U : nullptr, lowrank ? (int64_t)R * G * W : 0, es, false),
               span("state", state, B * (W - 1) * D, es, true),
               span("y", y, B * D, es, true)};
  if ((st = check_ptrs(s, 5)) != DSC_OK) return st;
  dsc::DecArgs a{};
  a.x = x; a.w = w; a.z = z; a.U = U; a.state = state; a.y = y;
  a.B = B; a.T = 1; a.D = D; a.W = W; a.H = H; a.R = R;
  a.bf16 = dtype == DSC_BF16;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.lowrank = lowrank;
  a.stream = stream;
  return hip_status(dsc::decode_launch(a));
}

dsc_status dsc_headwise_decode(const void *x, const void *w, void *state, void *y, int64_t B,
                               int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                               void *stream) {
  return decode_common(x, w, nullptr, nullptr, state, y, B, D, W, H, 0, dtype, flags, stream,
                       false);
}

dsc_status dsc_lowrank_decode(const void *x, const void *z, const void *U, void *state,
                              void *y, int64_t B, int64_t D, int W, int H, int R,
                              dsc_dtype dtype, unsigned flags, void *stream) {
  return decode_common(x, nullptr, z, U, state, y, B, D, W, H, R, dtype, flags, stream, true);
}

dsc_status dsc_decode_state(const void *x, void *state, int64_t B, int64_t T, int64_t D, int W,
                            dsc_dtype dtype, void *stream) {
  int V = 0;
  dsc_status st = check_common(B, T, D, W, 1, dtype, 0, &V);
  if (st != DSC_OK) return st;
  const int es = dtype == DSC_BF16 ? 2 : 4;
  Span s[2] = {span("x", x, B * T * D, es, false),
               span("state", state, B * (W - 1) * D, es, true)};
  if ((st = check_ptrs(s, 2)) != DSC_OK) return st;
  dsc::DecArgs a{};
  a.x = x; a.state = state;
  a.B = B; a.T = T; a.D = D; a.W = W; a.H = 1;
  a.bf16 = dtype == DSC_BF16;
  a.stream = stream;
  return hip_status(dsc::decode_state_launch(a));
}

static dsc_status static_check(int64_t B, int64_t T, int64_t D, int W, int H, dsc_dtype dtype,
                               unsigned flags) {
  int V = 0;
  dsc_status st = check_common(B, T, D, W, H, dtype, flags, &V);
  if (st != DSC_OK) return st;
  if (!headwise_h_ok(H, V))
    return fail(DSC_ERR_UNSUPPORTED,
                "H=%d: the static path needs H | %d or H = %d * m with m <= 64", H, V, V);
  return DSC_OK;
}

static dsc::StArgs static_args(int64_t B, int64_t T, int64_t D, int W, int H, dsc_dtype dtype,
                               unsigned flags, void *stream, bool bwd) {
  dsc::StArgs a{};
  a.B = B; a.T = T; a.D = D; a.W = W; a.H = H;
  a.bf16 = dtype == DSC_BF16;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.bwd = bwd;
  a.stream = stream;
  return a;
}

dsc_status dsc_static_fwd(const void *x, const void *w, void *y, int64_t B, int64_t T,
                          int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                          void *stream) {
  dsc_status st = static_check(B, T, D, W, H, dtype, flags);
  if (st != DSC_OK) return st;
  const int es = dtype == DSC_BF16 ? 2 : 4;
  const int64_t n_act = B * T * D, n_w = (D / H) * W;
  Span s[3] = {span("x", x, n_act, es, false), span("w", w, n_w, es, false),
               span("y", y, n_act, es, true)};
  if ((st = check_ptrs(s, 3)) != DSC_OK) return st;
  dsc::StArgs a = static_args(B, T, D, W, H, dtype, flags, stream, false);
  a.x = x; a.w = w; a.y = y;
  return hip_status(dsc::static_launch(a));
}

size_t dsc_static_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W, int H,
                                      dsc_dtype dtype) {
  if (static_check(B, T, D, W, H, dtype, 0) != DSC_OK) return 0;
  if (B == 0 || T == 0) return 0;
  return dsc::st_plan(B, T, D, W, H).bytes;
}

dsc_status dsc_static_bwd(const void *x, const void *w, const void *dy, void *dx, void *dw,
                          void *workspace, size_t workspace_bytes, int64_t B, int64_t T,
                          int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                          void *stream) {
  dsc_status st = static_check(B, T, D, W, H, dtype, flags);
  if (st != DSC_OK) return st;
  const int es = dtype == DSC_BF16 ? 2 : 4;
  const int64_t n_act = B * T * D, n_w = (D / H) * W;
  const size_t need = (B == 0 || T == 0) ? 0 : dsc::st_plan(B, T, D, W, H).bytes;
  if (need > 0 && workspace_bytes < need)
    return fail(DSC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu needed",
                workspace_bytes, need);
  if (need > 0 && workspace == nullptr)
    return fail(DSC_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  Span s[6] = {span("x", x, n_act, es, false),  span("w", w, n_w, es, false),
               span("dy", dy, n_act, es, false), span("dx", dx, n_act, es, true),
               span("dw", dw, n_w, es, true),
               span("workspace", workspace, (int64_t)need, 1, true)};
  if ((st = check_ptrs(s, 6)) != DSC_OK) return st;
  dsc::StArgs a = static_args(B, T, D, W, H, dtype, flags, stream, true);
  a.x = x; a.w = w; a.dy = dy; a.dx = dx; a.dw = dw; a.ws = workspace;
  return hip_status(dsc::static_launch(a));
}

dsc_status dsc_headwise_gen_fwd(const void *x, const void *xh, const void *Mt, void *y, int64_t B,
                                int64_t T, int64_t D, int64_t Dh, int W, int H,
                                dsc_dtype dtype, unsigned flags, void *stream) {
  int V = 0;
  dsc_status st = check_common(B, T, D, W, H, dtype, flags, &V);
  if (st != DSC_OK) return st;
  if (dtype != DSC_BF16) return fail(DSC_ERR_UNSUPPORTED, "generated filters: bf16 only");
  if (W != 1 && W != 2 && W != 4 && W != 8)
    return fail(DSC_ERR_UNSUPPORTED, "generated filters: W=%d not in {1, 2, 4, 8}", W);
  if (H % 8) return fail(DSC_ERR_UNSUPPORTED, "generated filters: H=%d not a multiple of 8", H);
  if (Dh < 64 || Dh % 64 || Dh > INT32_MAX)
    return fail(DSC_ERR_UNSUPPORTED, "generated filters: Dh=%lld not a positive multiple of 64",
                (long long)Dh);
  const int64_t GW = (D / H) * W;
  if (GW % 8)
    return fail(DSC_ERR_UNSUPPORTED, "generated filters: G*W=%lld not a multiple of 8",
                (long long)GW);
  if (B > 0 && T > 0 && B * T > kMaxElems / Dh)
    return fail(DSC_ERR_INVALID_ARG, "B*T*Dh exceeds 2^38 elements");
  const int64_t n_act = B * T * D;
  Span s[4] = {span("x", x, n_act, 2, false), span("xh", xh, B * T * Dh, 2, false),
               span("Mt", Mt, Dh * GW, 2, false), span("y", y, n_act, 2, true)};
  if ((st = check_ptrs(s, 4)) != DSC_OK) return st;
  dsc::GenArgs a{};
  a.x = x; a.xh = xh; a.Mt = Mt; a.y = y;
  a.B = B; a.T = T; a.D = D; a.Dh = Dh; a.W = W; a.H = H;
  a.residual = (flags & DSC_RESIDUAL) != 0;
  a.act = (flags & DSC_ACT_SILU) != 0;
  a.stream = stream;
  return hip_status(dsc::gen_launch(a));
}

}  // extern "C"
