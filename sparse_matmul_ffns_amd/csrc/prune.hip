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
#include "prep_bodies.hpp"

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
// nm_prune, 2:4 with 16-byte rows: each thread owns kPruneU 16-byte chunks (one group of four
// fp32 or two groups of bf16 each), all loaded before any is ranked, so that a thread keeps
// several loads in flight; the 2:4 choice is the extended-key network of select24.  I is the
// chunk index type (32-bit whenever the matrix has fewer than 2^32 chunks).
// ---------------------------------------------------------------------------
constexpr int kPruneU = 4;

template <typename T, typename I>
__global__ __launch_bounds__(256) void nm_prune24_vec_kernel(const T* __restrict__ A, int64_t lda, int64_t R,
                                                             int64_t K, uint8_t* __restrict__ mask,
                                                             int64_t ldmask) {
  constexpr int EPC = 16 / (int)sizeof(T);          // elements per chunk: 8 (bf16) or 4 (fp32)
  const I per_row = (I)(K / EPC);
  const I total = (I)R * per_row;
  const I base = (I)blockIdx.x * (256 * kPruneU) + threadIdx.x;
  u32x4 x[kPruneU];
  I rr[kPruneU], cc[kPruneU];
#pragma unroll
  for (int u = 0; u < kPruneU; ++u) {
    const I cid = base + 256 * u;
    rr[u] = cid / per_row;
    cc[u] = (cid - rr[u] * per_row) * EPC;
    if (cid < total)
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A + (int64_t)rr[u] * lda + cc[u]));
  }
#pragma unroll
  for (int u = 0; u < kPruneU; ++u) {
    if (base + 256 * u >= total) break;
    uint8_t* m = mask + (int64_t)rr[u] * ldmask + cc[u];
    if constexpr (sizeof(T) == 2) {
      uint32_t mw[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t lo = x[u][2 * g], hi = x[u][2 * g + 1];
        const uint32_t nib = select24_bf16(lo & 0xFFFFu, lo >> 16, hi & 0xFFFFu, hi >> 16);
        mw[g] = (1u << (8 * (nib & 3))) | (1u << (8 * (nib >> 2)));
      }
      *reinterpret_cast<u32x2*>(m) = u32x2{mw[0], mw[1]};
    } else {
      const uint32_t nib = select24(x[u][0] & 0x7FFFFFFFu, x[u][1] & 0x7FFFFFFFu, x[u][2] & 0x7FFFFFFFu,
                                    x[u][3] & 0x7FFFFFFFu);
      *reinterpret_cast<uint32_t*>(m) = (1u << (8 * (nib & 3))) | (1u << (8 * (nib >> 2)));
    }
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
                                                          int64_t meta_row, int32_t* bad_groups, int staged) {
  extern __shared__ __align__(16) unsigned char cst[];
  const int64_t chunks_per_row = (G + CG - 1) / CG;
  const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = R * chunks_per_row;
  // Staged loads (16-byte aligned rows): a thread's chunk is CG*M elements and CG*M mask bytes,
  // whole 16-byte pieces; the 64 lanes of a wave load the pieces of the wave's 64 chunks in order,
  // so that each load instruction covers whole lines, and hand them over through LDS.
  const int PA = CG * M * (int)sizeof(T) / 16, PM = CG * M / 16, PS = PA + PM;
  if (staged) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t K = G * M;
    for (int q = lane; q < 64 * PS; q += 64) {
      const int tl = q / PS, j = q % PS;
      const int64_t c = (int64_t)blockIdx.x * blockDim.x + 64 * wave + tl;
      int64_t rr = R - 1, gg = 0;
      if (c < total) {
        rr = c / chunks_per_row;
        gg = (c - rr * chunks_per_row) * CG;
      }
      u32x4 d;
      if (j < PA) {   // piece j of the chunk's elements; pieces past the row repeat its last one
        int64_t off = gg * M + (int64_t)j * (16 / (int)sizeof(T));
        if (off + 16 / (int)sizeof(T) > K) off = K - 16 / (int)sizeof(T);
        d = *reinterpret_cast<const u32x4*>(A + rr * lda + off);
      } else {        // piece j - PA of the chunk's mask bytes
        int64_t off = gg * M + (int64_t)(j - PA) * 16;
        if (off + 16 > K) off = K - 16;
        d = *reinterpret_cast<const u32x4*>(mask + rr * ldmask + off);
      }
      *reinterpret_cast<u32x4*>(cst + ((size_t)(64 * wave + tl) * PS + j) * 16) = d;
    }
    __syncthreads();
  }
  int bad = 0;
  if (cid < total) {
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
      if (staged) {
        const unsigned char* mine = cst + (size_t)threadIdx.x * PS * 16;
        __builtin_memcpy(xx, mine + (size_t)gi * M * sizeof(T), sizeof(T) * M);
        __builtin_memcpy(mm, mine + (size_t)PA * 16 + gi * M, M);
      } else {
#pragma unroll
        for (int p = 0; p < M; ++p) {
          mm[p] = mk[gi * M + p];
          xx[p] = a[gi * M + p];
        }
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
template <typename T, typename I>
__global__ __launch_bounds__(256) void nm_compress24_vec_kernel(const T* __restrict__ A, int64_t lda,
                                                                const uint8_t* __restrict__ mask, int64_t ldmask,
                                                                int64_t R, int64_t K, T* __restrict__ values,
                                                                uint8_t* __restrict__ meta, int32_t* bad_groups) {
  // each thread: kCompressU chunks of 16 elements (4 groups), all loaded before any is packed
  constexpr int kCompressU = 2;
  constexpr int NA = (int)sizeof(T);               // 16-byte loads of A per chunk (16 elements)
  const I per_row = (I)(K / 16);
  const I total = (I)R * per_row;
  const I base = (I)blockIdx.x * (256 * kCompressU) + threadIdx.x;
  u32x4 xa[kCompressU][NA], xm[kCompressU];
  I rr[kCompressU], cc[kCompressU];
#pragma unroll
  for (int u = 0; u < kCompressU; ++u) {
    const I cid = base + 256 * u;
    rr[u] = cid / per_row;
    cc[u] = (cid - rr[u] * per_row) * 16;
    if (cid < total) {
      const u32x4* a4 = reinterpret_cast<const u32x4*>(A + (int64_t)rr[u] * lda + cc[u]);
#pragma unroll
      for (int q = 0; q < NA; ++q) xa[u][q] = __builtin_nontemporal_load(a4 + q);
      xm[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(mask + (int64_t)rr[u] * ldmask + cc[u]));
    }
  }
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kCompressU; ++u) {
    if (base + 256 * u >= total) break;
    const int64_t r = rr[u], c0 = cc[u];
    uint32_t out[2 * NA];   // the 8 kept values of the chunk, packed
    uint32_t nibs = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // kept flags of the group as 4 bits: bit p set iff mask byte p is nonzero
      const uint32_t m32 = xm[u][g];
      const uint32_t nz = ((((m32 & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | m32) & 0x80808080u) >> 7;
      const uint32_t bits = (nz * 0x01020408u) >> 24;
      const bool ok = __builtin_popcount(bits) == 2;
      const uint32_t p0 = __builtin_ctz(bits | 0x10u) & 3u, p1 = (31 - __builtin_clz(bits | 1u)) & 3u;
      if (!ok) ++bad;
      // a group without exactly two survivors: positions 0 and 1, values +0.0
      nibs |= (ok ? (p0 | (p1 << 2)) : 0x4u) << (4 * g);
      if constexpr (sizeof(T) == 2) {
        // bytes 2p, 2p+1 of the pair (d23:d01) hold the group's value p
        const uint32_t d01 = xa[u][g >> 1][(g & 1) * 2], d23 = xa[u][g >> 1][(g & 1) * 2 + 1];
        const uint32_t sel = (p0 * 0x202u + 0x100u) | ((p1 * 0x202u + 0x100u) << 16);
        out[g] = ok ? __builtin_amdgcn_perm(d23, d01, sel) : 0u;
      } else {
        const u32x4 q = xa[u][g];
        auto pick = [&](uint32_t p) { return p == 0 ? q[0] : p == 1 ? q[1] : p == 2 ? q[2] : q[3]; };
        out[2 * g] = ok ? pick(p0) : 0u;
        out[2 * g + 1] = ok ? pick(p1) : 0u;
      }
    }
    T* vd = values + r * (K / 2) + c0 / 2;
#pragma unroll
    for (int q = 0; q < NA / 2; ++q)
      reinterpret_cast<u32x4*>(vd)[q] = u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
    *reinterpret_cast<uint16_t*>(meta + r * (K / 8) + c0 / 8) = (uint16_t)nibs;
  }
  if (bad_groups != nullptr && bad > 0) atomicAdd(bad_groups, bad);
}

// ---------------------------------------------------------------------------
// nm_prune_compress, 2:4 with 16-byte aligned rows: one pass (prep_bodies.hpp).
// ---------------------------------------------------------------------------
template <typename T, typename I>
__global__ __launch_bounds__(256) void nm_prune_compress24_vec_kernel(const T* __restrict__ A, int64_t lda,
                                                                      int64_t R, int64_t K,
                                                                      uint8_t* __restrict__ mask, int64_t ldmask,
                                                                      T* __restrict__ values,
                                                                      uint8_t* __restrict__ meta) {
  prune_compress24_body<T, I>(blockIdx.x, A, lda, R, K, mask, ldmask, values, meta);
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
  const int epc = 16 / esz;
  if (N == 2 && M == 4 && K % epc == 0 && (uintptr_t)A % 16 == 0 && (lda * esz) % 16 == 0 &&
      (uintptr_t)mask % (epc == 8 ? 8 : 4) == 0 && ldmask % (epc == 8 ? 8 : 4) == 0) {
    const int64_t n = R * (K / epc);
    if (n + 256 * kPruneU < (int64_t)UINT32_MAX)
      hipLaunchKernelGGL((nm_prune24_vec_kernel<T, uint32_t>), dim3(nblocks(n, 256 * kPruneU)), dim3(256), 0, s,
                         (const T*)A, lda, R, K, mask, ldmask);
    else
      hipLaunchKernelGGL((nm_prune24_vec_kernel<T, int64_t>), dim3(nblocks(n, 256 * kPruneU)), dim3(256), 0, s,
                         (const T*)A, lda, R, K, mask, ldmask);
    return hipGetLastError();
  }
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
    if (n + 512 < (int64_t)UINT32_MAX)
      hipLaunchKernelGGL((nm_compress24_vec_kernel<T, uint32_t>), dim3(nblocks(n, 512)), dim3(256), 0, s, (const T*)A,
                         lda, mask, ldmask, R, K, (T*)values, meta, bad);
    else
      hipLaunchKernelGGL((nm_compress24_vec_kernel<T, int64_t>), dim3(nblocks(n, 512)), dim3(256), 0, s, (const T*)A,
                         lda, mask, ldmask, R, K, (T*)values, meta, bad);
    return hipGetLastError();
  }
  const int64_t G = K / M;
  const int CG = compress_chunk_groups(N, M);
  const int64_t meta_row = meta_row_bytes(K, N, M);
  const int64_t n = R * ((G + CG - 1) / CG);
  // staged loads when rows are 16-byte aligned and whole 16-byte pieces (so is every clamped piece)
  const int staged = K % 16 == 0 && (uintptr_t)A % 16 == 0 && ((int64_t)lda * (int64_t)sizeof(T)) % 16 == 0 &&
                     (uintptr_t)mask % 16 == 0 && ldmask % 16 == 0 && !force_generic();
  const size_t lds = staged ? (size_t)256 * (CG * M * sizeof(T) / 16 + CG * M / 16) * 16 : 0;
  if (lds > 0) {
    (void)hipFuncSetAttribute((const void*)nm_compress_kernel<T, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)nm_compress_kernel<T, 8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)nm_compress_kernel<T, 16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  }
  switch (M) {
    case 4:
      hipLaunchKernelGGL((nm_compress_kernel<T, 4>), dim3(nblocks(n, 256)), dim3(256), lds, s, (const T*)A, lda,
                         mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad, staged);
      break;
    case 8:
      hipLaunchKernelGGL((nm_compress_kernel<T, 8>), dim3(nblocks(n, 256)), dim3(256), lds, s, (const T*)A, lda,
                         mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad, staged);
      break;
    default:
      hipLaunchKernelGGL((nm_compress_kernel<T, 16>), dim3(nblocks(n, 256)), dim3(256), lds, s, (const T*)A,
                         lda, mask, ldmask, R, G, N, CG, (T*)values, meta, meta_row, bad, staged);
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

// ---------------------------------------------------------------------------
// nm_prune_compress for bf16 N:8 (1 <= N <= 7) with 16-byte aligned rows and K % 64 == 0, one pass:
// one thread per chunk of CG groups whose positions fill whole bytes (CG = 4 for even N, 8 for
// odd).  The 64 lanes of a wave load the pieces of the wave's 64 chunks in address order (whole
// lines per instruction) into LDS, each thread's region padded by 16 bytes so that the lanes'
// reads of their own chunks fall on distinct banks.  Per group the positions are ranked on keys
// extended by position ((|x| << 3) | (7 - p): distinct, larger key first, lower position on ties,
// the order of rank_of) -- the N largest are those at least the N-th of the keys sorted by a
// 19-comparator network -- and the kept ones taken in ascending order from the kept bits; the chunk
// leaves as 16-byte stores of mask bytes and values and byte stores of its positions.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void nm_prune_compress_m8_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                                   int64_t R, int64_t K, uint8_t* __restrict__ mask,
                                                                   int64_t ldmask, uint16_t* __restrict__ values,
                                                                   uint8_t* __restrict__ meta) {
  constexpr int M = 8, CG = (N % 2 == 0) ? 4 : 8, E = CG * M, PA = E * 2 / 16, PS = PA + 1;
  constexpr int MB = CG * N * 3 / 8;           // metadata bytes per chunk
  constexpr int NW32 = (CG * N * 3 + 31) / 32; // 32-bit words of positions
  __shared__ u32x4 stage[256 * PS];
  const int64_t G = K / M, per_row = G / CG, total = R * per_row;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int q = lane; q < 64 * PA; q += 64) {
    const int tl = q / PA, j = q % PA;
    const int64_t c = (int64_t)blockIdx.x * 256 + 64 * wave + tl;
    if (c < total) {
      const int64_t rr = c / per_row, gg = (c - rr * per_row) * CG;
      stage[(64 * wave + tl) * PS + j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A + rr * lda + gg * M + 8 * j));
    }
  }
  __syncthreads();
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int64_t rr = c / per_row, gg = (c - rr * per_row) * CG;
  uint32_t x[E / 2];
#pragma unroll
  for (int j = 0; j < PA; ++j) {
    const u32x4 v = stage[threadIdx.x * PS + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * j + e] = v[e];
  }
  uint32_t mk[E / 4];          // mask bytes, 4 per word
  uint32_t vo[CG * N / 2];     // kept values, 2 per word
  uint32_t w[NW32];            // positions, LSB first
#pragma unroll
  for (int k = 0; k < NW32; ++k) w[k] = 0;
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    uint32_t ext[M];
#pragma unroll
    for (int p = 0; p < M; ++p) {
      const uint32_t b = (x[(g * M + p) >> 1] >> (16 * (p & 1))) & 0x7FFFu;
      ext[p] = (b << 3) | (uint32_t)(7 - p);
    }
    // the N-th largest extended key (a sorting network over a copy, descending), then position p
    // is kept iff its key is at least that one (the keys are distinct)
    uint32_t srt[M];
#pragma unroll
    for (int p = 0; p < M; ++p) srt[p] = ext[p];
    auto cx = [&](int i, int j) {
      const uint32_t hi = srt[i] > srt[j] ? srt[i] : srt[j], lo = srt[i] > srt[j] ? srt[j] : srt[i];
      srt[i] = hi;
      srt[j] = lo;
    };
    // 8-input sorting network of 19 comparators
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 4); cx(3, 6);
    cx(1, 2); cx(3, 4); cx(5, 6);
    const uint32_t thr = srt[N - 1];
    uint32_t kept = 0;
#pragma unroll
    for (int p = 0; p < M; ++p) kept |= (ext[p] >= thr ? 1u : 0u) << p;
    // mask bytes of the group: byte p = bit p of kept
    mk[2 * g] = ((kept & 1u) | ((kept & 2u) << 7) | ((kept & 4u) << 14) | ((kept & 8u) << 21));
    mk[2 * g + 1] = (((kept >> 4) & 1u) | (((kept >> 4) & 2u) << 7) | (((kept >> 4) & 4u) << 14) |
                     (((kept >> 4) & 8u) << 21));
    uint32_t rest = kept;
#pragma unroll
    for (int s2 = 0; s2 < N; ++s2) {
      const uint32_t p = (uint32_t)__builtin_ctz(rest);
      rest &= rest - 1u;
      const uint32_t d = (p >> 1) == 0 ? x[4 * g] : (p >> 1) == 1 ? x[4 * g + 1] : (p >> 1) == 2 ? x[4 * g + 2] : x[4 * g + 3];
      const uint32_t v = (d >> (16 * (p & 1))) & 0xFFFFu;
      const int i = g * N + s2;   // kept value index within the chunk
      if (i & 1) vo[i >> 1] |= v << 16;
      else vo[i >> 1] = v;
      const int off = 3 * i;
      w[off >> 5] |= p << (off & 31);
      if ((off & 31) > 29) w[(off >> 5) + 1] |= p >> (32 - (off & 31));
    }
  }
  u32x4* md = reinterpret_cast<u32x4*>(mask + rr * ldmask + gg * M);
#pragma unroll
  for (int k = 0; k < E / 16; ++k) md[k] = u32x4{mk[4 * k], mk[4 * k + 1], mk[4 * k + 2], mk[4 * k + 3]};
  u32x4* vd = reinterpret_cast<u32x4*>(values + rr * (G * N) + gg * N);
#pragma unroll
  for (int k = 0; k < CG * N / 8; ++k) vd[k] = u32x4{vo[4 * k], vo[4 * k + 1], vo[4 * k + 2], vo[4 * k + 3]};
  uint8_t* mt = meta + rr * (G * N * 3 / 8) + (gg / CG) * MB;
#pragma unroll
  for (int k = 0; k < MB; ++k) mt[k] = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
}

template <typename T>
static hipError_t prune_compress_dispatch(const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                          uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta, hipStream_t s) {
  const int esz = sizeof(T);
  if (N == 2 && M == 4 && K % 16 == 0 && (uintptr_t)A % 16 == 0 && (lda * esz) % 16 == 0 &&
      (uintptr_t)mask % 16 == 0 && ldmask % 16 == 0 && (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 2 == 0) {
    const int64_t n = R * (K / 16);
    if (n + 256 * kFusedU < (int64_t)UINT32_MAX)
      hipLaunchKernelGGL((nm_prune_compress24_vec_kernel<T, uint32_t>), dim3(nblocks(n, 256 * kFusedU)), dim3(256), 0,
                         s, (const T*)A, lda, R, K, mask, ldmask, (T*)values, meta);
    else
      hipLaunchKernelGGL((nm_prune_compress24_vec_kernel<T, int64_t>), dim3(nblocks(n, 256 * kFusedU)), dim3(256), 0,
                         s, (const T*)A, lda, R, K, mask, ldmask, (T*)values, meta);
    return hipGetLastError();
  }
  if (esz == 2 && M == 8 && K % 64 == 0 && (uintptr_t)A % 16 == 0 && (lda * esz) % 16 == 0 &&
      (uintptr_t)mask % 16 == 0 && ldmask % 16 == 0 && (uintptr_t)values % 16 == 0 && !force_generic()) {
    const int64_t chunks = R * ((K / 8) / (N % 2 == 0 ? 4 : 8));
    const unsigned grid = (unsigned)((chunks + 255) / 256);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, (const uint16_t*)A, lda, R, K, mask, ldmask,
                         (uint16_t*)values, meta);
      return hipGetLastError();
    };
    switch (N) {
      case 1: return go(nm_prune_compress_m8_kernel<1>);
      case 2: return go(nm_prune_compress_m8_kernel<2>);
      case 3: return go(nm_prune_compress_m8_kernel<3>);
      case 4: return go(nm_prune_compress_m8_kernel<4>);
      case 5: return go(nm_prune_compress_m8_kernel<5>);
      case 6: return go(nm_prune_compress_m8_kernel<6>);
      default: return go(nm_prune_compress_m8_kernel<7>);
    }
  }
  // other patterns and layouts: the two passes, mask in between
  const hipError_t e = prune_dispatch<T>(A, lda, R, K, N, M, mask, ldmask, s);
  if (e != hipSuccess) return e;
  return compress_dispatch<T>(A, lda, mask, ldmask, R, K, N, M, values, meta, nullptr, s);
}

hipError_t launch_nm_prune_compress(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                    uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta, hipStream_t s) {
  return dt == DT_BF16 ? prune_compress_dispatch<uint16_t>(A, lda, R, K, N, M, mask, ldmask, values, meta, s)
                       : prune_compress_dispatch<uint32_t>(A, lda, R, K, N, M, mask, ldmask, values, meta, s);
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
