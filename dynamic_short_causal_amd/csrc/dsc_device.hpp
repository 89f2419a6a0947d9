// dsc_device.hpp -- device helpers shared by the gfx950 kernels of libdsc:
// 16-byte vector loads and stores of bf16 / fp32 activations with fp32
// unpacking, small contiguous filter-row loads, round-to-nearest-even bf16
// packing (v_cvt_pk_bf16_f32 on gfx950) and the SiLU epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsc {

typedef uint16_t bf16;  // storage type of bfloat16 tensors

// Elements per 16-byte vector.
template <typename E> struct Vw;
template <> struct Vw<float> { static constexpr int n = 4; };
template <> struct Vw<bf16> { static constexpr int n = 8; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// ---- one 16-byte vector of activations -----------------------------------
__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void st16(void *p, uint4 v) {
  *reinterpret_cast<uint4 *>(p) = v;
}
// Non-temporal (streaming) forms.  Which streams of a kernel take them is a
// measured choice: on MI355X a kernel runs fastest when part of its streams
// are non-temporal, and slower when all or none are.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16nt(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16nt(void *p, uint4 v) {
  const u32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t *>(p));
}

template <typename E> __device__ __forceinline__ void unpack(uint4 r, float (&o)[Vw<E>::n]);
template <> __device__ __forceinline__ void unpack<float>(uint4 r, float (&o)[4]) {
  o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y);
  o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
}
template <> __device__ __forceinline__ void unpack<bf16>(uint4 r, float (&o)[8]) {
  o[0] = bf_lo(r.x); o[1] = bf_hi(r.x); o[2] = bf_lo(r.y); o[3] = bf_hi(r.y);
  o[4] = bf_lo(r.z); o[5] = bf_hi(r.z); o[6] = bf_lo(r.w); o[7] = bf_hi(r.w);
}

template <typename E> __device__ __forceinline__ uint4 pack(const float (&o)[Vw<E>::n]);
template <> __device__ __forceinline__ uint4 pack<float>(const float (&o)[4]) {
  return make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                    __float_as_uint(o[3]));
}
template <> __device__ __forceinline__ uint4 pack<bf16>(const float (&o)[8]) {
  return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                    pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
}

// ---- a short contiguous row of N elements (filter taps) -------------------
// The row starts at a multiple of N elements from a 16-byte aligned base, so
// it is aligned to gcd(N * sizeof(E), 16) bytes; the widest such access is
// used.  Raw bits are returned in `r` (up to 8 dwords) and unpacked later, so
// the load can be issued early.
template <typename E, int N> struct RowBits {
  static constexpr int bytes = N * (int)sizeof(E);
  static constexpr int dwords = (bytes + 3) / 4;
  uint32_t d[dwords > 0 ? dwords : 1];
};

// NTL: non-temporal loads (the 16- and 8-byte forms)
template <typename E, int N, bool NTL = false>
__device__ __forceinline__ RowBits<E, N> ld_row(const E *p) {
  RowBits<E, N> r;
  constexpr int bytes = N * (int)sizeof(E);
  if constexpr (bytes % 16 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 16; ++i) {
      const uint4 v = NTL ? ld16nt(reinterpret_cast<const uint4 *>(p) + i)
                          : reinterpret_cast<const uint4 *>(p)[i];
      r.d[4 * i] = v.x; r.d[4 * i + 1] = v.y; r.d[4 * i + 2] = v.z; r.d[4 * i + 3] = v.w;
    }
  } else if constexpr (bytes % 8 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 8; ++i) {
      uint2 v;
      if constexpr (NTL) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p) + i);
        v = make_uint2(t.x, t.y);
      } else {
        v = reinterpret_cast<const uint2 *>(p)[i];
      }
      r.d[2 * i] = v.x; r.d[2 * i + 1] = v.y;
    }
  } else if constexpr (bytes % 4 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 4; ++i) r.d[i] = reinterpret_cast<const uint32_t *>(p)[i];
  } else {
    // odd number of bf16 elements: 2-byte accesses
    const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
    for (int i = 0; i < RowBits<E, N>::dwords; ++i) {
      uint32_t lo = q[2 * i];
      uint32_t hi = (2 * i + 1 < N) ? (uint32_t)q[2 * i + 1] : 0u;
      r.d[i] = lo | (hi << 16);
    }
  }
  return r;
}

template <typename E, int N>
__device__ __forceinline__ void unpack_row(const RowBits<E, N> &r, float (&o)[N]) {
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = __uint_as_float(r.d[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = (i & 1) ? bf_hi(r.d[i >> 1]) : bf_lo(r.d[i >> 1]);
  }
}

// Store N fp32 values as a contiguous row of E (same alignment rule as ld_row).
template <typename E, int N>
__device__ __forceinline__ void st_row(E *p, const float (&o)[N]) {
  constexpr int bytes = N * (int)sizeof(E);
  uint32_t d[(bytes + 3) / 4 > 0 ? (bytes + 3) / 4 : 1];
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = __float_as_uint(o[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) d[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
    if constexpr (N & 1) d[N / 2] = pack_bf16x2(o[N - 1], 0.f);
  }
  if constexpr (bytes % 16 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 16; ++i)
      reinterpret_cast<uint4 *>(p)[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
  } else if constexpr (bytes % 8 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 8; ++i)
      reinterpret_cast<uint2 *>(p)[i] = make_uint2(d[2 * i], d[2 * i + 1]);
  } else if constexpr (bytes % 4 == 0) {
#pragma unroll
    for (int i = 0; i < bytes / 4; ++i) reinterpret_cast<uint32_t *>(p)[i] = d[i];
  } else {
    uint16_t *q = reinterpret_cast<uint16_t *>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = (uint16_t)((i & 1) ? (d[i >> 1] >> 16) : (d[i >> 1] & 0xffffu));
  }
}

// ---- SiLU epilogue ---------------------------------------------------------
// sigma(s) = 1 / (1 + e^-s) via the hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoid_f(float s) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-s));
}
__device__ __forceinline__ float silu_f(float s) { return s * sigmoid_f(s); }
// d/ds [s sigma(s)] = sigma(s) (1 + s (1 - sigma(s)))
__device__ __forceinline__ float silu_grad_f(float s) {
  float sg = sigmoid_f(s);
  return sg * (1.0f + s * (1.0f - sg));
}

// ---- filter-gradient sum over the lanes of one group ------------------------
// A filter group of L >= 1 lanes occupies an aligned run of L consecutive
// lanes (lane % L is the lane's place in its group; the wave holds 64 / L
// whole groups, any lanes past them idle).  After the call the group's first
// lane holds the sum of a[j] over the group.  L a power of two: xor butterfly,
// every lane of the group ends with the sum.  Otherwise a halving tree inside
// the group: in round s (1, 2, 4, ...) a lane adds the value s lanes up if
// that lane is still in its group, which leaves the first lane with the sum
// of all L.
template <int N>
__device__ __forceinline__ void group_sum(float (&a)[N], int L, int lane_in_group) {
  if ((L & (L - 1)) == 0) {
    for (int m = 1; m < L; m <<= 1)
#pragma unroll
      for (int j = 0; j < N; ++j) a[j] += __shfl_xor(a[j], m);
  } else {
    for (int s = 1; s < L; s <<= 1) {
      const bool in = lane_in_group + s < L;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float o = __shfl_down(a[j], s);
        a[j] += in ? o : 0.f;
      }
    }
  }
}

}  // namespace dsc
