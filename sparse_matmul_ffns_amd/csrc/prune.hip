// Magnitude N:M pruning, compression and decompression (gfx950).
//
// Pruning rule ("Success story: ESPLAG", Highlights and Solution; "To 2:4
// Sparsity and Beyond", abstract): keep the N largest magnitudes of every M
// consecutive elements along K, the lower position winning ties.  Magnitudes
// are compared as the bit pattern without its sign, which orders finite values
// exactly like |x| (and +0.0 equal to -0.0).
//
// All three kernels are HBM-bound streaming passes: one thread owns a chunk of
// whole groups that starts on a 16-byte boundary of the input row when the
// caller's layout allows (vec != 0), so that loads and stores are dwordx4 and
// consecutive lanes touch consecutive bytes.
#include "common.hpp"
#include "launch.hpp"

namespace nms {

// ---------------------------------------------------------------------------
// nm_prune: one thread per chunk of E = max(M, 16 / sizeof(T)) elements.
// ---------------------------------------------------------------------------
template <typename T, int M>
__global__ __launch_bounds__(256) void nm_prune_kernel(const T* __restrict__ A, int64_t lda, int64_t R,
                                                       int64_t K, int N, uint8_t* __restrict__ mask,
                                                       int64_t ldmask, int vec) {
  constexpr int E = (M * (int)sizeof(T) >= 16) ? M : 16 / (int)sizeof(T);
  const int64_t chunks_per_row = (K + E - 1) / E;
  const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (cid >= R * chunks_per_row) return;
  const int64_t r = cid / chunks_per_row;
  const int64_t c0 = (cid - r * chunks_per_row) * E;
  const T* a = A + r * lda + c0;
  uint8_t* m = mask + r * ldmask + c0;
  T x[E];
  const bool full = c0 + E <= K;
  if (vec && full) {
    const u32x4* a4 = reinterpret_cast<const u32x4*>(a);
#pragma unroll
    for (int i = 0; i < E * (int)sizeof(T) / 16; ++i) {
      u32x4 t = __builtin_nontemporal_load(a4 + i);
      __builtin_memcpy(&x[i * 16 / sizeof(T)], &t, 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = (c0 + i < K) ? a[i] : (T)0;
  }
  uint8_t out[E];
#pragma unroll
  for (int g = 0; g < E / M; ++g) {
    uint32_t k[M];
#pragma unroll
    for (int p = 0; p < M; ++p) k[p] = Elem<T>::key(x[g * M + p]);
#pragma unroll
    for (int p = 0; p < M; ++p) out[g * M + p] = rank_of<M>(k, p) < N ? 1 : 0;
  }
  if (vec && full) {
    if constexpr (E == 4) {
      uint32_t t; __builtin_memcpy(&t, out, 4); *reinterpret_cast<uint32_t*>(m) = t;
    } else if constexpr (E == 8) {
      uint64_t t; __builtin_memcpy(&t, out, 8); *reinterpret_cast<uint64_t*>(m) = t;
    } else {
#pragma unroll
      for (int i = 0; i < E / 16; ++i) {
        u32x4 t; __builtin_memcpy(&t, out + 16 * i, 16); reinterpret_cast<u32x4*>(m)[i] = t;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (c0 + i < K) m[i] = out[i];
  }
}

// ---------------------------------------------------------------------------
// Bit-stream writer/reader for the packed positions of one row segment that
// starts on a byte boundary.
// ---------------------------------------------------------------------------
struct BitWriter {
  uint8_t* dst;
  uint32_t acc = 0;
  int nbits = 0;
  __device__ explicit BitWriter(uint8_t* d) : dst(d) {}
  __device__ inline void put(uint32_t v, int b) {
    acc |= v << nbits;
    nbits += b;
    while (nbits >= 8) {
      *dst++ = (uint8_t)(acc & 0xFF);
      acc >>= 8;
      nbits -= 8;
    }
  }
  __device__ inline void flush() {
    if (nbits > 0) *dst++ = (uint8_t)(acc & 0xFF);
    acc = 0;
    nbits = 0;
  }
};

struct BitReader {
  const uint8_t* src;
  uint32_t acc = 0;
  int nbits = 0;
  __device__ explicit BitReader(const uint8_t* s) : src(s) {}
  __device__ inline uint32_t get(int b) {
    while (nbits < b) {
      acc |= (uint32_t)(*src++) << nbits;
      nbits += 8;
    }
    uint32_t v = acc & ((1u << b) - 1u);
    acc >>= b;
    nbits -= b;
    return v;
  }
};

// Groups per thread: a whole number of bytes of metadata, at least 4 groups.
__host__ __device__ inline int compress_chunk_groups(int N, int M) {
  int b = 1;
  while ((1 << b) < M) ++b;
  const int gb = N * b;
  int g = gb, e = 8;  // gcd(gb, 8)
  while (e) { int t = g % e; g = e; e = t; }
  const int base = 8 / g;
  return base < 4 ? 4 : base;
}

// ---------------------------------------------------------------------------
// nm_compress: one thread per chunk of CG groups of one row.
// ---------------------------------------------------------------------------
template <typename T, int M>
__global__ __launch_bounds__(256) void nm_compress_kernel(const T* __restrict__ A, int64_t lda,
                                                          const uint8_t* __restrict__ mask, int64_t ldmask,
                                                          int64_t R, int64_t G, int N, int CG,
                                                          T* __restrict__ values, uint8_t* __restrict__ meta,
                                                          int64_t meta_row, int32_t* bad_groups) {
  const int64_t chunks_per_row = (G + CG - 1) / CG;
  const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int bad = 0;
  if (cid < R * chunks_per_row) {
    const int64_t r = cid / chunks_per_row;
    const int64_t g0 = (cid - r * chunks_per_row) * CG;
    const int ng = (int)((G - g0) < CG ? (G - g0) : CG);
    const int b = ceil_log2(M);
    const T* a = A + r * lda + g0 * M;
    const uint8_t* mk = mask + r * ldmask + g0 * M;
    T* v = values + r * G * N + g0 * N;
    BitWriter bw(meta + r * meta_row + (g0 * N * b) / 8);
    for (int gi = 0; gi < ng; ++gi) {
      uint8_t mm[M];
      T xx[M];
#pragma unroll
      for (int p = 0; p < M; ++p) {
        mm[p] = mk[gi * M + p];
        xx[p] = a[gi * M + p];
      }
      int cnt = 0;
#pragma unroll
      for (int p = 0; p < M; ++p) cnt += mm[p] ? 1 : 0;
      if (cnt != N) {
        ++bad;
        for (int s = 0; s < N; ++s) {
          v[gi * N + s] = (T)0;
          bw.put((uint32_t)s, b);
        }
      } else {
        int s = 0;
#pragma unroll
        for (int p = 0; p < M; ++p) {
          if (mm[p]) {
            v[gi * N + s] = xx[p];
            bw.put((uint32_t)p, b);
            ++s;
          }
        }
      }
    }
    bw.flush();
  }
  if (bad_groups != nullptr && bad > 0) atomicAdd(bad_groups, bad);
}

// ---------------------------------------------------------------------------
// nm_compress, 2:4 with 16-byte aligned rows: one thread per 16 elements
// (4 groups): 16-byte loads of A and mask, one 16- or 32-byte store of the 8
// kept values and one 2-byte store of their 4 nibbles.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void nm_compress24_vec_kernel(const T* __restrict__ A, int64_t lda,
                                                                const uint8_t* __restrict__ mask, int64_t ldmask,
                                                                int64_t R, int64_t K, T* __restrict__ values,
                                                                uint8_t* __restrict__ meta, int32_t* bad_groups) {
  const int64_t per_row = K / 16;
  const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int bad = 0;
  if (cid < R * per_row) {
    const int64_t r = cid / per_row;
    const int64_t c0 = (cid - r * per_row) * 16;
    T x[16];
    uint8_t m[16];
    const u32x4* a4 = reinterpret_cast<const u32x4*>(A + r * lda + c0);
#pragma unroll
    for (int i = 0; i < 16 * (int)sizeof(T) / 16; ++i) {
      u32x4 t = __builtin_nontemporal_load(a4 + i);
      __builtin_memcpy(&x[i * 16 / sizeof(T)], &t, 16);
    }
    {
      u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(mask + r * ldmask + c0));
      __builtin_memcpy(m, &t, 16);
    }
    T v[8];
    uint32_t nibs = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      int cnt = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p) cnt += m[4 * g + p] ? 1 : 0;
      uint32_t nib = 0;
      T v0 = (T)0, v1 = (T)0;
      if (cnt == 2) {
        int s = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (m[4 * g + p]) {
            if (s == 0) v0 = x[4 * g + p]; else v1 = x[4 * g + p];
            nib |= (uint32_t)p << (2 * s);
            ++s;
          }
        }
      } else {
        ++bad;
        nib = 0x4;  // positions 0 and 1, values +0.0
      }
      v[2 * g] = v0;
      v[2 * g + 1] = v1;
      nibs |= nib << (4 * g);
    }
    T* vd = values + r * (K / 2) + c0 / 2;
#pragma unroll
    for (int i = 0; i < 8 * (int)sizeof(T) / 16; ++i) {
      u32x4 t;
      __builtin_memcpy(&t, &v[i * 16 / sizeof(T)], 16);
      __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(vd) + i);
    }
    *reinterpret_cast<uint16_t*>(meta + r * (K / 8) + c0 / 8) = (uint16_t)nibs;
  }
  if (bad_groups != nullptr && bad > 0) atomicAdd(bad_groups, bad);
}

// ---------------------------------------------------------------------------
// nm_decompress: one thread per chunk of CG groups of one row.
// ---------------------------------------------------------------------------
template <typename T, int M>
__global__ __launch_bounds__(256) void nm_decompress_kernel(const T* __restrict__ values,
                                                            const uint8_t* __restrict__ meta, int64_t R,
                                                            int64_t G, int N, int CG, int64_t meta_row,
                                                            T* __restrict__ out, int64_t lda) {
  const int64_t chunks_per_row = (G + CG - 1) / CG;
  const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (cid >= R * chunks_per_row) return;
  const int64_t r = cid / chunks_per_row;
  const int64_t g0 = (cid - r * chunks_per_row) * CG;
  const int ng = (int)((G - g0) < CG ? (G - g0) : CG);
  const int b = ceil_log2(M);
  const T* v = values + r * G * N + g0 * N;
  T* o = out + r * lda + g0 * M;
  BitReader br(meta + r * meta_row + (g0 * N * b) / 8);
  for (int gi = 0; gi < ng; ++gi) {
    T xx[M];
#pragma unroll
    for (int p = 0; p < M; ++p) xx[p] = (T)0;
    for (int s = 0; s < N; ++s) {
      const uint32_t p = br.get(b);
      xx[p & (M - 1)] = v[gi * N + s];
    }
#pragma unroll
    for (int p = 0; p < M; ++p) o[gi * M + p] = xx[p];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline unsigned nblocks(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

template <typename T>
static hipError_t prune_dispatch(const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                 uint8_t* mask, int64_t ldmask, hipStream_t s) {
  const int esz = sizeof(T);
  auto run = [&](auto kern, int E) {
    const int mask_al = E < 16 ? E : 16;
    const int vec = ((uintptr_t)A % 16 == 0) && ((lda * esz) % 16 == 0) &&
                    ((uintptr_t)mask % mask_al == 0) && (ldmask % mask_al == 0);
    const int64_t n = R * ((K + E - 1) / E);
    hipLaunchKernelGGL(kern, dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)A, lda, R, K, N, mask,
                       ldmask, vec);
    return hipGetLastError();
  };
  const int E4 = 4 * esz >= 16 ? 4 : 16 / esz, E8 = 8 * esz >= 16 ? 8 : 16 / esz, E16 = 16;
  switch (M) {
    case 4: return run(nm_prune_kernel<T, 4>, E4);
    case 8: return run(nm_prune_kernel<T, 8>, E8);
    default: return run(nm_prune_kernel<T, 16>, E16);
  }
}

hipError_t launch_nm_prune(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                           uint8_t* mask, int64_t ldmask, hipStream_t s) {
  return dt == DT_BF16 ? prune_dispatch<uint16_t>(A, lda, R, K, N, M, mask, ldmask, s)
                       : prune_dispatch<uint32_t>(A, lda, R, K, N, M, mask, ldmask, s);
}

template <typename T>
static hipError_t compress_dispatch(const void* A, int64_t lda, const uint8_t* mask, int64_t ldmask,
                                    int64_t R, int64_t K, int N, int M, void* values, uint8_t* meta,
                                    int32_t* bad, hipStream_t s) {
  const int esz = sizeof(T);
  if (N == 2 && M == 4 && K % 16 == 0 && (uintptr_t)A % 16 == 0 && (lda * esz) % 16 == 0 &&
      (uintptr_t)mask % 16 == 0 && ldmask % 16 == 0 && (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 2 == 0) {
    const int64_t n = R * (K / 16);
    hipLaunchKernelGGL(nm_compress24_vec_kernel<T>, dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)A, lda, mask,
                       ldmask, R, K, (T*)values, meta, bad);
    return hipGetLastError();
  }
  const int64_t G = K / M;
  const int CG = compress_chunk_groups(N, M);
  const int64_t meta_row = meta_row_bytes(K, N, M);
  const int64_t n = R * ((G + CG - 1) / CG);
  switch (M) {
    case 4:
      hipLaunchKernelGGL((nm_compress_kernel<T, 4>), dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)A, lda,
                         mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad);
      break;
    case 8:
      hipLaunchKernelGGL((nm_compress_kernel<T, 8>), dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)A, lda,
                         mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad);
      break;
    default:
      hipLaunchKernelGGL((nm_compress_kernel<T, 16>), dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)A,
                         lda, mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_nm_compress(int dt, const void* A, int64_t lda, const uint8_t* mask, int64_t ldmask,
                              int64_t R, int64_t K, int N, int M, void* values, uint8_t* meta, int32_t* bad,
                              hipStream_t s) {
  return dt == DT_BF16 ? compress_dispatch<uint16_t>(A, lda, mask, ldmask, R, K, N, M, values, meta, bad, s)
                       : compress_dispatch<uint32_t>(A, lda, mask, ldmask, R, K, N, M, values, meta, bad, s);
}

template <typename T>
static hipError_t decompress_dispatch(const void* values, const uint8_t* meta, int64_t R, int64_t K, int N,
                                      int M, void* out, int64_t lda, hipStream_t s) {
  const int64_t G = K / M;
  const int CG = compress_chunk_groups(N, M);
  const int64_t meta_row = meta_row_bytes(K, N, M);
  const int64_t n = R * ((G + CG - 1) / CG);
  switch (M) {
    case 4:
      hipLaunchKernelGGL((nm_decompress_kernel<T, 4>), dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)values,
                         meta, R, G, N, CG, meta_row, (T*)out, lda);
      break;
    case 8:
      hipLaunchKernelGGL((nm_decompress_kernel<T, 8>), dim3(nblocks(n, 256)), dim3(256), 0, s, (const T*)values,
                         meta, R, G, N, CG, meta_row, (T*)out, lda);
      break;
    default:
      hipLaunchKernelGGL((nm_decompress_kernel<T, 16>), dim3(nblocks(n, 256)), dim3(256), 0, s,
                         (const T*)values, meta, R, G, N, CG, meta_row, (T*)out, lda);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_nm_decompress(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N,
                                int M, void* out, int64_t lda, hipStream_t s) {
  return dt == DT_BF16 ? decompress_dispatch<uint16_t>(values, meta, R, K, N, M, out, lda, s)
                       : decompress_dispatch<uint32_t>(values, meta, R, K, N, M, out, lda, s);
}

}  // namespace nms
