// stream_ceiling.hip -- a plain streaming kernel for measuring what HBM
// bandwidth a given mix of reads and writes reaches on this GPU.  It is the
// yardstick the convolution kernels are compared with, not part of the
// convolution: libdsc_stream.so is loaded by the benchmark's ceiling mode only.
//
// dsc_stream_mix reads up to three input tensors and writes up to two output
// tensors in one sweep, so one launch moves the bytes of one convolution
// call.  The largest tensor has n 16-byte vectors; a tensor of n >> s vectors
// (s = its shift) is addressed at index i >> s, so 2^s neighbouring lanes
// share one of its vectors, the way neighbouring lanes of the head-wise
// kernels share one filter row.  Each thread takes UNR vectors of a grid-
// stride sweep.  Loads have no branch (an index past the end is clamped to
// the last vector); an output vector is written by the first lane of its
// 2^s-lane group, as the xor of the inputs plus the output number, with the
// non-temporal loads and stores the convolution kernels use.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kMaxT = 3;  // tensors per side
constexpr int UNR = 4;    // vectors per thread per sweep step

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Mix {
  const u32x4 *in[kMaxT];
  u32x4 *out[kMaxT];
  int in_shift[kMaxT], out_shift[kMaxT];
  int64_t n;      // vectors of the largest tensor
  u32x4 *sink;    // read-only mixes: written only if an xor equals `key`, so
  unsigned key;   // the loads cannot be dropped
};

template <int NIN, int NOUT>
__global__ __launch_bounds__(1024) void stream_kernel(Mix m) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * UNR;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * UNR + threadIdx.x; base < m.n;
       base += stride) {
    u32x4 acc[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
      u32x4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t i = min(base + (int64_t)u * blockDim.x, m.n - 1);
        v[u] = __builtin_nontemporal_load(m.in[k] + (i >> m.in_shift[k]));
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) acc[u] ^= v[u];
    }
    if constexpr (NOUT == 0) {
      u32x4 r = acc[0];
#pragma unroll
      for (int u = 1; u < UNR; ++u) r ^= acc[u];
      if ((r.x ^ r.y ^ r.z ^ r.w) == m.key) *m.sink = r;
    }
#pragma unroll
    for (int k = 0; k < NOUT; ++k)
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int64_t i = base + (int64_t)u * blockDim.x;
        const int64_t mask = ((int64_t)1 << m.out_shift[k]) - 1;
        if (i < m.n && (i & mask) == 0)
          __builtin_nontemporal_store(acc[u] + (unsigned)k, m.out[k] + (i >> m.out_shift[k]));
      }
  }
}

template <int NIN>
hipError_t launch_out(const Mix &m, int nout, int grid, int block, hipStream_t s) {
  switch (nout) {
    case 0: hipLaunchKernelGGL((stream_kernel<NIN, 0>), dim3(grid), dim3(block), 0, s, m); break;
    case 1: hipLaunchKernelGGL((stream_kernel<NIN, 1>), dim3(grid), dim3(block), 0, s, m); break;
    case 2: hipLaunchKernelGGL((stream_kernel<NIN, 2>), dim3(grid), dim3(block), 0, s, m); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

// n_vec: 16-byte vectors of the largest tensor, a multiple of 2^shift for
// every tensor; in_shift/out_shift: log2 of how many times smaller each
// tensor is (tensor k holds n_vec >> shift[k] vectors).  A read-only mix
// (nout = 0) needs `sink`, 16 device bytes written only when the xor of the
// loaded data equals `key`.  Pointers are device pointers, 16-byte aligned.  Returns 0 on success, -1 for bad
// arguments, else the HIP error code.
int dsc_stream_mix(const void *const *in, const int *in_shift, int nin, void *const *out,
                   const int *out_shift, int nout, int64_t n_vec, int grid, int block,
                   void *sink, unsigned key, void *stream) {
  if (nin < 0 || nin > kMaxT || nout < 0 || nout > 2 || nin + nout == 0 || n_vec < 1) return -1;
  if (nout == 0 && (!sink || ((uintptr_t)sink & 15))) return -1;
  if (grid < 1 || block < 64 || block > 1024 || block % 64) return -1;
  Mix m{};
  m.n = n_vec;
  m.sink = reinterpret_cast<u32x4 *>(sink);
  m.key = key;
  for (int k = 0; k < nin; ++k) {
    if (!in[k] || ((uintptr_t)in[k] & 15) || in_shift[k] < 0 || in_shift[k] > 6) return -1;
    if (n_vec % ((int64_t)1 << in_shift[k])) return -1;
    m.in[k] = reinterpret_cast<const u32x4 *>(in[k]);
    m.in_shift[k] = in_shift[k];
  }
  for (int k = 0; k < nout; ++k) {
    if (!out[k] || ((uintptr_t)out[k] & 15) || out_shift[k] < 0 || out_shift[k] > 6) return -1;
    if (n_vec % ((int64_t)1 << out_shift[k])) return -1;
    m.out[k] = reinterpret_cast<u32x4 *>(out[k]);
    m.out_shift[k] = out_shift[k];
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (nin) {
    case 0: e = launch_out<0>(m, nout, grid, block, s); break;
    case 1: e = launch_out<1>(m, nout, grid, block, s); break;
    case 2: e = launch_out<2>(m, nout, grid, block, s); break;
    default: e = launch_out<3>(m, nout, grid, block, s); break;
  }
  return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
