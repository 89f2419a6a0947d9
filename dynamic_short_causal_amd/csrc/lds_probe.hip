// lds_probe.hip -- how gfx950's LDS serves one wave's access for a given
// per-lane address pattern: the clock cost of a 16- or 8-byte read, a
// transposing 8-byte read, or a 16-, 8- or 2-byte write, with 8 waves per CU
// issuing the same pattern back to back.  It is the evidence behind the LDS
// layouts of the kernels (the granule swizzle of the generated-filter GEMM,
// the vector order of the low-rank rings), not part of the convolution:
// libdsc_ldsprobe.so is loaded by the benchmark's --lds-banks mode only.
//
// dsc_lds_probe(offsets, op, clocks): offsets holds 64 byte offsets (lane i
// accesses LDS at offsets[i]), each a multiple of the access size and below
// 16 KiB.  Every wave issues 8 accesses per iteration at offsets[lane] + 2 KiB
// * k (k = 0..7, which keeps the bank of every lane) for 256 iterations; the
// result is the median over 256 workgroups (one per CU) of the workgroup's
// clock64() span divided by the workgroup's access instructions (8 waves x
// 256 x 8).  Returns 0, a HIP error code, or -1 for a bad argument.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBlocks = 256, kThreads = 512, kIters = 256, kLds = 65536;

// OP: 0 read 16 B, 1 read 8 B, 2 transposing read 8 B, 3 write 16 B, 4 write 8 B, 5 write 2 B
template <int OP>
__global__ __launch_bounds__(kThreads) void lds_probe_kernel(const unsigned *tab,
                                                             unsigned long long *out, int *sink) {
  __shared__ __align__(16) unsigned char lds[kLds];
  for (int i = threadIdx.x; i < kLds / 4; i += kThreads) reinterpret_cast<int *>(lds)[i] = i;
  // the array's address escapes into an asm statement, so that its memory
  // clobbers keep every store (nothing reads them back otherwise)
  asm volatile("" ::"v"((unsigned)(uintptr_t)lds) : "memory");
  __syncthreads();
  // waves alternate between two 16 KiB halves (a multiple of the bank turn)
  const unsigned off = tab[threadIdx.x & 63] + ((threadIdx.x >> 6) & 1) * 16384u;
  uint4 acc = make_uint4(threadIdx.x, 0, 0, 0);
  __syncthreads();
  const unsigned long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      unsigned o = off + k * 2048 + (it & 1) * 1024;
      asm volatile("" : "+v"(o));  // one instruction per access (no merged pairs)
      unsigned char *a = lds + o;
      if constexpr (OP == 0) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a);
        acc.x ^= v.x; acc.y ^= v.y; acc.z ^= v.z; acc.w ^= v.w;
      } else if constexpr (OP == 1) {
        const uint2 v = *reinterpret_cast<const uint2 *>(a);
        acc.x ^= v.x; acc.y ^= v.y;
      } else if constexpr (OP == 2) {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(__attribute__((address_space(3))) char *)(uintptr_t)a);
        acc.x ^= (unsigned)(unsigned short)v[0] | ((unsigned)(unsigned short)v[1] << 16);
        acc.y ^= (unsigned)(unsigned short)v[2] | ((unsigned)(unsigned short)v[3] << 16);
      } else if constexpr (OP == 3) {
        *reinterpret_cast<uint4 *>(a) = acc;
        acc.x += 1;
      } else if constexpr (OP == 4) {
        *reinterpret_cast<uint2 *>(a) = make_uint2(acc.x, acc.y);
        acc.x += 1;
      } else {
        *reinterpret_cast<unsigned short *>(a) = (unsigned short)acc.x;
        acc.x += 1;
      }
    }
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  const unsigned long long t1 = clock64();
  if (threadIdx.x == 0) out[blockIdx.x] = t1 - t0;
  // a condition on every lane of acc the reads fill keeps the reads
  const bool hit = OP == 0 ? acc.x == 0x7fffffffu && acc.y == 3u && acc.z == 5u && acc.w == 7u
                           : acc.x == 0x7fffffffu && acc.y == 3u;
  if (hit) sink[0] = 1;
}

template <int OP> hipError_t launch(const unsigned *tab, unsigned long long *out, int *sink) {
  hipLaunchKernelGGL(lds_probe_kernel<OP>, dim3(kBlocks), dim3(kThreads), 0, 0, tab, out, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" int dsc_lds_probe(const unsigned *offsets, int op, double *clocks) {
  static const unsigned size[6] = {16, 8, 8, 16, 8, 2};
  if (!offsets || !clocks || op < 0 || op > 5) return -1;
  for (int i = 0; i < 64; ++i)
    if (offsets[i] % size[op] || offsets[i] + size[op] > 16384) return -1;
  unsigned *tab = nullptr;
  unsigned long long *out = nullptr;
  int *sink = nullptr;
  hipError_t e = hipMalloc(&tab, 64 * sizeof(unsigned));
  if (e == hipSuccess) e = hipMalloc(&out, kBlocks * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMalloc(&sink, sizeof(int));
  if (e == hipSuccess) e = hipMemcpy(tab, offsets, 64 * sizeof(unsigned), hipMemcpyHostToDevice);
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {  // the first launch warms up
    switch (op) {
      case 0: e = launch<0>(tab, out, sink); break;
      case 1: e = launch<1>(tab, out, sink); break;
      case 2: e = launch<2>(tab, out, sink); break;
      case 3: e = launch<3>(tab, out, sink); break;
      case 4: e = launch<4>(tab, out, sink); break;
      default: e = launch<5>(tab, out, sink); break;
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  std::vector<unsigned long long> h(kBlocks);
  if (e == hipSuccess)
    e = hipMemcpy(h.data(), out, kBlocks * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    std::sort(h.begin(), h.end());
    *clocks = (double)h[kBlocks / 2] / (8.0 * kIters * 8);
  }
  if (tab) (void)hipFree(tab);
  if (out) (void)hipFree(out);
  if (sink) (void)hipFree(sink);
  return e == hipSuccess ? 0 : (int)e;
}
