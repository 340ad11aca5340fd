// Device helpers shared by the gfx950 kernels of the N:M sparse FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

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

// The same rank over fp64 keys (the V:N:M column norms).
template <int M>
__device__ inline int rank_f64(const double (&k)[M], int p) {
  int r = 0;
#pragma unroll
  for (int q = 0; q < M; ++q) {
    r += (k[q] > k[p]) ? 1 : 0;
    r += (q < p && k[q] == k[p]) ? 1 : 0;
  }
  return r;
}

// 2:4 selection on four keys: returns the nibble p0 | p1 << 2 (p0 < p1) of the two positions
// with rank < 2 under rank_of.  Each key is extended by its position, (k << 2) | (3 - p), so
// that the extended keys are distinct and order exactly like rank_of (larger key first, then
// lower position); the two largest extended keys are found with three max/min pairs.
template <typename K>
__device__ inline uint32_t select24_ext(K c0, K c1, K c2, K c3) {
  const K m01 = c0 > c1 ? c0 : c1, n01 = c0 > c1 ? c1 : c0;
  const K m23 = c2 > c3 ? c2 : c3, n23 = c2 > c3 ? c3 : c2;
  const K t1 = m01 > m23 ? m01 : m23;
  const K lo = m01 > m23 ? m23 : m01, hi_n = n01 > n23 ? n01 : n23;
  const K t2 = lo > hi_n ? lo : hi_n;
  const uint32_t pa = 3u - (uint32_t)(t1 & 3), pb = 3u - (uint32_t)(t2 & 3);
  const uint32_t p0 = pa < pb ? pa : pb, p1 = pa < pb ? pb : pa;
  return p0 | (p1 << 2);
}
// 32-bit extended keys: the largest and second largest of c0..c3 (the second largest of four is
// the median of {max(c0,c1,c2), med(c0,c1,c2), c3}); the compiler maps these to the 3-input
// max / median instructions.
__device__ inline uint32_t umax2(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ inline uint32_t umin2(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ inline uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return umax2(umin2(a, b), umin2(umax2(a, b), c));
}
__device__ inline uint32_t select24_ext32(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  const uint32_t m3 = umax2(umax2(c0, c1), c2);
  const uint32_t d3 = umed3(c0, c1, c2);
  const uint32_t t1 = umax2(m3, c3);
  const uint32_t t2 = umed3(m3, d3, c3);
  const uint32_t pa = (~t1) & 3u, pb = (~t2) & 3u;
  const uint32_t p0 = pa < pb ? pa : pb, p1 = pa < pb ? pb : pa;
  return p0 | (p1 << 2);
}
__device__ inline uint32_t select24(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  if ((k0 | k1 | k2 | k3) < (1u << 30))
    return select24_ext32((k0 << 2) | 3u, (k1 << 2) | 2u, (k2 << 2) | 1u, k3 << 2);
  return select24_ext<uint64_t>(((uint64_t)k0 << 2) | 3u, ((uint64_t)k1 << 2) | 2u, ((uint64_t)k2 << 2) | 1u,
                                (uint64_t)k3 << 2);
}
// The same selection on four raw bf16 patterns (the sign bit is shifted out of the key).
__device__ inline uint32_t select24_bf16(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return select24_ext32((b0 << 17) | 3u, (b1 << 17) | 2u, (b2 << 17) | 1u, b3 << 17);
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

// Column-panel-major, XCD-aware tile order.  The dispatcher deals consecutive workgroup ids to
// the 8 XCDs in turn, and each XCD's L2 serves only its own CUs.  When the ntn column panels
// divide evenly among the XCDs, XCD x takes panels x*pp .. x*pp + pp - 1 (pp = ntn / 8) for every
// row tile, so each column panel of the dense operand is fetched into one L2 only; its slots are
// ordered in groups of gm row tiles x pp panels (the tiles that run together share both operands'
// panels).  Otherwise the plain XCD-contiguous order grouped by gm row tiles.
__device__ inline void panel_major_tile(int wg_hw, int ntm, int ntn, int gm, int& tm, int& tn) {
  const int nx = 8;
  if (ntn % nx == 0) {
    const int pp = ntn / nx;
    const int x = wg_hw % nx, slot = wg_hw / nx;
    const int grp = slot / (gm * pp);
    const int first_m = grp * gm;
    const int gsz = (ntm - first_m) < gm ? (ntm - first_m) : gm;
    const int within = slot - grp * gm * pp;
    tm = first_m + within % gsz;
    tn = x * pp + within / gsz;
    return;
  }
  const int wg = xcd_remap(wg_hw, ntm * ntn);
  const int grp = wg / (gm * ntn);
  const int first_m = grp * gm;
  const int gsz = (ntm - first_m) < gm ? (ntm - first_m) : gm;
  const int within = wg - grp * gm * ntn;
  tm = first_m + within % gsz;
  tn = within / gsz;
}

// fp32 -> bf16 with round to nearest, ties to even (the bf16 result keeps the fp32 sign and
// exponent and the top 7 stored significand bits, rounded on the 16 dropped ones); NaN stays a
// quiet NaN, values past the bf16 range round to infinity.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
// Eight fp32 values (a, then b) as two bf16x8 parts: hi holds the top 16 bits of each value (the
// value truncated), lo the remainder rounded to nearest even, so hi + lo keeps about 16
// significant bits of a finite value.  Products of bf16 operands with both parts, summed in fp32,
// carry an fp32 operand through bf16 matrix instructions.
__device__ inline void split_bf16x8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  u32x4 h, l;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b0 = __float_as_uint(v[2 * q]), b1 = __float_as_uint(v[2 * q + 1]);
    const uint32_t t0 = b0 & 0xFFFF0000u, t1 = b1 & 0xFFFF0000u;
    h[q] = (b0 >> 16) | t1;
    l[q] = (uint32_t)f32_to_bf16_rne(v[2 * q] - __uint_as_float(t0)) |
           ((uint32_t)f32_to_bf16_rne(v[2 * q + 1] - __uint_as_float(t1)) << 16);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}
// One output element of a product: fp32 as is, bf16 rounded to nearest even.
__device__ inline void store_out(float* p, float v) { *p = v; }
__device__ inline void store_out(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// Host-side knob, read on every call: NMSPARSE_FORCE_GENERIC=1 makes every call take its
// plain SIMT kernel instead of the tiled ones (the tests compare the two).
inline bool env_is_one(const char* name) {
  const char* e = getenv(name);
  return e && e[0] == '1';
}
inline bool force_generic() { return env_is_one("NMSPARSE_FORCE_GENERIC"); }

}  // namespace nms
