// stream_ceiling.hip -- plain streaming kernels for measuring what HBM
// bandwidth a given mix of reads and writes, and a given access order,
// reaches on this GPU.  It is the
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

// ---------------------------------------------------------------------------
// Access order.  The same bytes as the head-wise forward (x and a filter
// tensor a quarter of its size read, y written; 2 lanes share one 8-byte
// filter load) moved in three geometries, with no arithmetic:
//   mode 0, long strips: a lane walks `len` tokens of one 16-byte column,
//     loading 4 ahead; 256-lane workgroups cover 256 columns of one chunk;
//   mode 1, short chunks in address order: a wave takes `len` tokens of a
//     64-column strip, loaded at once; the `nw` waves of a workgroup take
//     consecutive chunks of that strip; workgroups run strip-fastest;
//   mode 2, whole rows: a workgroup moves `len` whole token rows in turn.
// x and y hold rows * ncol 16-byte vectors (ncol a multiple of 256), the
// filter tensor rows * ncol / 4.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void ao_strips(const u32x4 *__restrict__ x, const uint2 *__restrict__ w,
                                                 u32x4 *__restrict__ y, int T, int ncol, int len,
                                                 int nchunk) {
  int bid = blockIdx.x;
  const int nvb = ncol / 256;
  const int vb = bid % nvb;
  bid /= nvb;
  const int chunk = bid % nchunk, b = bid / nchunk;
  const int v = vb * 256 + (int)threadIdx.x;
  const int t0 = chunk * len, t1 = min(T, t0 + len);
  const int64_t r0 = (int64_t)b * T;
  for (int t = t0; t < t1; t += 4) {
    u32x4 xr[4];
    uint2 wr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (t + u < t1) {
        xr[u] = __builtin_nontemporal_load(x + (r0 + t + u) * ncol + v);
        const uint2 *wp = w + ((r0 + t + u) * ncol + v) / 2;
        wr[u] = *wp;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (t + u < t1) {
        u32x4 o = xr[u];
        o.x ^= wr[u].x;
        o.y ^= wr[u].y;
        __builtin_nontemporal_store(o, y + (r0 + t + u) * ncol + v);
      }
  }
}
template <int LEN>
__global__ __launch_bounds__(512) void ao_chunks(const u32x4 *__restrict__ x, const uint2 *__restrict__ w,
                                                  u32x4 *__restrict__ y, int T, int ncol, int nw,
                                                  int nchunk) {
  int bid = blockIdx.x;
  const int nstrip = ncol / 64;
  const int strip = bid % nstrip;
  bid /= nstrip;
  const int cgs = (nchunk + nw - 1) / nw;
  const int cg = bid % cgs, b = bid / cgs;
  const int chunk = cg * nw + (int)(threadIdx.x >> 6);
  if (chunk >= nchunk) return;
  const int v = strip * 64 + (int)(threadIdx.x & 63);
  const int t0 = chunk * LEN, t1 = min(T, t0 + LEN);
  const int64_t r0 = (int64_t)b * T;
  u32x4 xr[LEN];
  uint2 wr[LEN];
#pragma unroll
  for (int u = 0; u < LEN; ++u)
    if (t0 + u < t1) {
      xr[u] = __builtin_nontemporal_load(x + (r0 + t0 + u) * ncol + v);
      wr[u] = *(w + ((r0 + t0 + u) * ncol + v) / 2);
    }
#pragma unroll
  for (int u = 0; u < LEN; ++u)
    if (t0 + u < t1) {
      u32x4 o = xr[u];
      o.x ^= wr[u].x;
      o.y ^= wr[u].y;
      __builtin_nontemporal_store(o, y + (r0 + t0 + u) * ncol + v);
    }
}
__global__ __launch_bounds__(256) void ao_rows(const u32x4 *__restrict__ x, const uint2 *__restrict__ w,
                                               u32x4 *__restrict__ y, int64_t rows, int ncol, int len) {
  const int64_t r0 = (int64_t)blockIdx.x * len, r1 = min(rows, r0 + len);
  const int64_t n = (r1 - r0) * ncol;
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    u32x4 xr[4];
    uint2 wr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + 256 * u;
      if (j < n) {
        xr[u] = __builtin_nontemporal_load(x + r0 * ncol + j);
        wr[u] = *(w + (r0 * ncol + j) / 2);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + 256 * u;
      if (j < n) {
        u32x4 o = xr[u];
        o.x ^= wr[u].x;
        o.y ^= wr[u].y;
        __builtin_nontemporal_store(o, y + r0 * ncol + j);
      }
    }
  }
}
}  // namespace

extern "C" {

// One launch of the access-order probe above.  x, w, y: device pointers
// (16-byte aligned) of B*T*ncol, B*T*ncol/4 and B*T*ncol 16-byte vectors;
// ncol a multiple of 256; mode 0: len >= 1 tokens per lane; mode 1: len 4
// tokens per wave, nw 1..8 waves per workgroup; mode 2: len >= 1 rows per
// workgroup.  Returns 0 on success, -1 for bad arguments, else the HIP error.
int dsc_stream_order(const void *x, const void *w, void *y, int B, int T, int ncol, int mode,
                     int len, int nw, void *stream) {
  if (!x || !w || !y || B < 1 || T < 1 || ncol < 256 || ncol % 256 || len < 1) return -1;
  hipStream_t s = (hipStream_t)stream;
  const u32x4 *xp = reinterpret_cast<const u32x4 *>(x);
  const uint2 *wp = reinterpret_cast<const uint2 *>(w);
  u32x4 *yp = reinterpret_cast<u32x4 *>(y);
  if (mode == 0) {
    const int nchunk = (T + len - 1) / len;
    hipLaunchKernelGGL(ao_strips, dim3((unsigned)((int64_t)B * nchunk * (ncol / 256))), dim3(256),
                       0, s, xp, wp, yp, T, ncol, len, nchunk);
  } else if (mode == 1) {
    if (len != 4 || nw < 1 || nw > 8) return -1;
    const int nchunk = (T + len - 1) / len;
    const int64_t grid = (int64_t)B * ((nchunk + nw - 1) / nw) * (ncol / 64);
    hipLaunchKernelGGL(ao_chunks<4>, dim3((unsigned)grid), dim3(64 * nw), 0, s, xp, wp, yp, T,
                       ncol, nw, nchunk);
  } else if (mode == 2) {
    const int64_t rows = (int64_t)B * T;
    hipLaunchKernelGGL(ao_rows, dim3((unsigned)((rows + len - 1) / len)), dim3(256), 0, s, xp, wp,
                       yp, rows, ncol, len);
  } else {
    return -1;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
