// Device helpers shared by the gfx950 kernels of the N:M sparse FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nms {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw storage of one element: bf16 is kept as its 16-bit pattern, fp32 as its
// 32-bit pattern.  Selection only ever compares magnitudes, and values are
// copied bit for bit, so the kernels never need the arithmetic type except in
// the products.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int bytes = 2;
  // |x| ordering of finite values == unsigned ordering of the bits without sign
  __device__ static inline uint32_t key(uint16_t b) { return b & 0x7FFFu; }
  __device__ static inline float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
  __device__ static inline bool positive(uint16_t b) { return !(b & 0x8000u) && (b & 0x7FFFu) != 0 && (b & 0x7FFFu) <= 0x7F80u; }
};
template <> struct Elem<uint32_t> {
  static constexpr int bytes = 4;
  __device__ static inline uint32_t key(uint32_t b) { return b & 0x7FFFFFFFu; }
  __device__ static inline float to_f32(uint32_t b) { return __uint_as_float(b); }
  __device__ static inline bool positive(uint32_t b) { return !(b & 0x80000000u) && (b & 0x7FFFFFFFu) != 0 && (b & 0x7FFFFFFFu) <= 0x7F800000u; }
};

// Rank of position p among the M keys of a group: keys strictly larger, plus
// equal keys at lower positions.  Position p is kept iff rank < N.
template <int M>
__device__ inline int rank_of(const uint32_t (&k)[M], int p) {
  int r = 0;
#pragma unroll
  for (int q = 0; q < M; ++q) {
    r += (k[q] > k[p]) ? 1 : 0;
    r += (q < p && k[q] == k[p]) ? 1 : 0;
  }
  return r;
}

// 2:4 selection on four keys: returns the nibble p0 | p1 << 2 (p0 < p1).
__device__ inline uint32_t select24(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  uint32_t k[4] = {k0, k1, k2, k3};
  uint32_t nib = 0;
  int s = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (rank_of<4>(k, p) < 2) {
      nib |= (uint32_t)p << (2 * s);
      ++s;
    }
  }
  return nib;
}

__device__ inline int ceil_log2(int m) {
  int b = 0;
  while ((1 << b) < m) ++b;
  return b < 1 ? 1 : b;
}

// XCD-aware remap of a linear workgroup id: consecutive hardware ids are
// dealt round-robin to the 8 XCDs, so give each XCD a contiguous range of
// logical tiles (neighbouring tiles then share that XCD's L2).
__device__ inline int xcd_remap(int wg, int nwg) {
  const int nx = 8;
  if (nwg % nx != 0) return wg;
  const int per = nwg / nx;
  return (wg % nx) * per + (wg / nx);
}

}  // namespace nms
