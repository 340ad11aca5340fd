// V:N:M (VENOM-style) pruning and compression in one HBM pass (gfx950).
//
// "To 2:4 Sparsity and Beyond" (abstract) prunes FFN activations to v:n:m;
// "Success story: ESPLAG" (Solution) stores them in the VENOM format; ReLU as
// the activation comes from "Sparser, Faster, Lighter Transformer Language
// Models" (Methodologie).  The rule implemented: per V-row block and M-column
// group keep the 4 columns with the largest block L1 norm, then per row the
// 2 largest magnitudes among those 4.
//
// One workgroup owns one V-row block and CW columns.  It stages the tile in
// LDS once (ReLU applied on the way in), so HBM is read exactly once:
//   1. coalesced 16-byte loads of the V x CW tile into LDS;
//   2. one lane per column adds |h| over the V rows in fp64, top to bottom
//      (the same sequence of additions as a sequential loop, so the sums are
//      bit-identical to any other implementation that adds in row order);
//   3. one lane per group ranks the M sums (lower column wins ties) and
//      writes the group's 4 column indices;
//   4. one lane per (row, 4 groups) picks 2 of the 4 selected values and
//      writes 4 x 2 values (16 bytes for bf16) and 16 bits of nibbles.
#include "common.hpp"
#include "launch.hpp"

namespace nms {

// Chunks of 16 bytes per thread and tile on the streaming path (a 64 KB tile, 256 threads).
constexpr int kStreamChunks = 16;

template <typename T, int M>
__global__ __launch_bounds__(256) void venom_prune_kernel(const T* __restrict__ Z, int64_t ldz, int64_t K, int V,
                                                          int relu, int CW, T* __restrict__ values,
                                                          uint8_t* __restrict__ meta, uint8_t* __restrict__ colsel,
                                                          uint8_t* __restrict__ mask, int64_t ldmask, int vec_in,
                                                          int vec_out, int ntx, int64_t ntiles, int stream) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int EPC = 16 / sizeof(T);       // elements per 16-byte chunk
  const int tid = threadIdx.x;
  const int64_t G = K / M;
  const int pitch = CW + 8;   // elements per LDS row: 16 bytes of padding spread the rows over the banks
  T* tile = reinterpret_cast<T*>(smem);
  double* l1 = reinterpret_cast<double*>(smem + (size_t)V * pitch * sizeof(T));
  uint8_t* csel = reinterpret_cast<uint8_t*>(l1 + CW);
  const int cpr = CW / EPC;
  const int nch = V * cpr;

  auto relu_chunk = [&](u32x4 t) {
    if (relu) {
      T x[EPC];
      __builtin_memcpy(x, &t, 16);
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[e] = Elem<T>::positive(x[e]) ? x[e] : (T)0;
      __builtin_memcpy(&t, x, 16);
    }
    return t;
  };
  // streaming path: full aligned 64 KB tiles; the next tile's chunks are loaded into registers
  // while the current tile is ranked and written out
  u32x4 pre[kStreamChunks];
  auto load_tile = [&](int64_t t) {
    const int64_t b = t / ntx;
    const T* zb = Z + b * V * ldz + (t - b * ntx) * CW;
#pragma unroll
    for (int u = 0; u < kStreamChunks; ++u) {
      const int i = tid + 256 * u;
      const int r = i / cpr, c = (i - r * cpr) * EPC;
      pre[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zb + (int64_t)r * ldz + c));
    }
  };
  if (stream && (int64_t)blockIdx.x < ntiles) load_tile(blockIdx.x);

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
  const int64_t blk = t / ntx;
  const int64_t c0 = (t - blk * ntx) * CW;
  const int cols = (int)((K - c0) < CW ? (K - c0) : CW);  // valid columns in this tile (multiple of M)
  const int ngr = cols / M;                                // valid groups

  // 1. stage the tile (ReLU'd) in LDS
  if (stream) {
#pragma unroll
    for (int u = 0; u < kStreamChunks; ++u) {
      const int i = tid + 256 * u;
      const int r = i / cpr, c = (i - r * cpr) * EPC;
      *reinterpret_cast<u32x4*>(tile + r * pitch + c) = relu_chunk(pre[u]);
    }
    if (t + gridDim.x < ntiles) load_tile(t + gridDim.x);
  } else {
    const T* zb = Z + blk * V * ldz + c0;
    for (int i = tid; i < nch; i += 256) {
      const int r = i / cpr, c = (i - r * cpr) * EPC;
      u32x4 v;
      if (vec_in && c + EPC <= cols) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zb + (int64_t)r * ldz + c));
      } else {
        T x[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[e] = (c + e < cols) ? zb[(int64_t)r * ldz + c + e] : (T)0;
        __builtin_memcpy(&v, x, 16);
      }
      *reinterpret_cast<u32x4*>(tile + r * pitch + c) = relu_chunk(v);
    }
  }
  __syncthreads();

  // 2. block column L1 norms, fp64, rows in ascending order.  bf16 tiles of 512 columns: a lane
  //    owns two adjacent columns and reads both with one 4-byte LDS load per row (8 rows at a
  //    time), the two sums being independent chains; otherwise one column per lane
  if (sizeof(T) == 2 && cols == 512) {
    for (int c = 2 * tid; c < cols; c += 512) {   // cols is a multiple of M, hence even
      double a0 = 0.0, a1 = 0.0;
      const unsigned char* col = reinterpret_cast<const unsigned char*>(tile) + 2 * c;
      int r = 0;
      for (; r + 8 <= V; r += 8) {
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = *reinterpret_cast<const uint32_t*>(col + (size_t)(r + k) * pitch * 2);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          a0 += (double)__uint_as_float((w[k] & 0x7FFFu) << 16);
          a1 += (double)__uint_as_float(w[k] & 0x7FFF0000u);
        }
      }
      for (; r < V; ++r) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(col + (size_t)r * pitch * 2);
        a0 += (double)__uint_as_float((w & 0x7FFFu) << 16);
        a1 += (double)__uint_as_float(w & 0x7FFF0000u);
      }
      l1[c] = a0;
      l1[c + 1] = a1;
    }
  } else {
    for (int c = tid; c < cols; c += 256) {
      double acc = 0.0;
      int r = 0;
      for (; r + 8 <= V; r += 8) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = fabsf(Elem<T>::to_f32(tile[(r + k) * pitch + c]));
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += (double)x[k];
      }
      for (; r < V; ++r) acc += (double)fabsf(Elem<T>::to_f32(tile[r * pitch + c]));
      l1[c] = acc;
    }
  }
  __syncthreads();

  // 3. keep the 4 columns of each group with the largest L1 (lower column on ties): one lane per
  //    (group, column) ranks its column among the group's M (M consecutive lanes of a wave hold a
  //    group); the group's first lane packs the kept columns, in ascending order, from the wave's
  //    ballot
  for (int u = tid; u < ngr * M; u += 256) {   // ngr * M == cols; 256 is a multiple of M
    const int g = u / M, p = u % M;
    const double kp = l1[u];
    int rk = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const double kq = l1[g * M + q];
      rk += (kq > kp || (q < p && kq == kp)) ? 1 : 0;
    }
    const uint64_t kept = __ballot(rk < 4);
    if (p == 0) {
      const uint32_t bits = (uint32_t)(kept >> ((threadIdx.x & 63) & ~(M - 1))) & ((1u << M) - 1u);
      uint32_t packed = 0, rest = bits;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        packed |= (uint32_t)__builtin_ctz(rest) << (8 * j);
        rest &= rest - 1u;
      }
      *reinterpret_cast<uint32_t*>(csel + 4 * g) = packed;
      const int64_t gg = c0 / M + g;
      uint8_t* dst = colsel + (blk * G + gg) * 4;
      if (((uintptr_t)dst & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = packed;
      } else {
        for (int e = 0; e < 4; ++e) dst[e] = (uint8_t)(packed >> (8 * e));
      }
    }
  }
  __syncthreads();

  // 4. per row, 2 of the 4 selected columns of each group
  const int nq = (ngr + 3) / 4;
  const int64_t meta_row = (G + 1) / 2;
  if (sizeof(T) == 2 && !mask && vec_out && ngr % 4 == 0 && 256 % nq == 0) {
    // Fast path: a lane keeps one quad of groups (q) for the whole tile and walks rows; the LDS
    // offsets of its 16 selected columns are computed once.
    const int q = tid % nq, rstep = 256 / nq;
    int ofs[4][4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * q + gi;
      const uint32_t cs = *reinterpret_cast<const uint32_t*>(csel + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) ofs[gi][j] = g * M + (int)((cs >> (8 * j)) & 0xFF);
    }
    const int64_t gglob = c0 / M + 4 * q;
    for (int r = tid / nq; r < V; r += rstep) {
      const uint16_t* trow = reinterpret_cast<const uint16_t*>(tile) + r * pitch;
      uint32_t out[4];
      uint32_t nibs = 0;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        uint32_t x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = trow[ofs[gi][j]];
        const uint32_t nib = select24_bf16(x[0], x[1], x[2], x[3]);
        const uint32_t d01 = x[0] | (x[1] << 16), d23 = x[2] | (x[3] << 16);
        const uint32_t j0 = nib & 3, j1 = nib >> 2;
        // bytes 2j, 2j+1 of the pair (d23:d01) hold value j
        const uint32_t sel = (j0 * 0x202u + 0x100u) | ((j1 * 0x202u + 0x100u) << 16);
        out[gi] = __builtin_amdgcn_perm(d23, d01, sel);
        nibs |= nib << (4 * gi);
      }
      const int64_t row = blk * V + r;
      *reinterpret_cast<u32x4*>(values + row * (G * 2) + gglob * 2) = u32x4{out[0], out[1], out[2], out[3]};
      uint8_t* md = meta + row * meta_row + gglob / 2;
      if (((uintptr_t)md & 1) == 0) {
        *reinterpret_cast<uint16_t*>(md) = (uint16_t)nibs;
      } else {
        md[0] = (uint8_t)(nibs & 0xFF);
        md[1] = (uint8_t)(nibs >> 8);
      }
    }
  } else
  for (int u = tid; u < V * nq; u += 256) {
    const int r = u / nq, q = u - r * nq;
    const int64_t row = blk * V + r;
    T v[8];
    uint32_t nibs = 0;
    const int gq = (ngr - 4 * q) < 4 ? (ngr - 4 * q) : 4;
    uint8_t msk[4][M];
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * q + gi;
      if (gi < gq) {
        const uint32_t cs = *reinterpret_cast<const uint32_t*>(csel + 4 * g);
        T x[4];
        uint32_t k[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = tile[r * pitch + g * M + ((cs >> (8 * j)) & 0xFF)];
          k[j] = Elem<T>::key(x[j]);
        }
        const uint32_t nib = select24(k[0], k[1], k[2], k[3]);
        const int j0 = nib & 3, j1 = (nib >> 2) & 3;
        v[2 * gi] = x[j0];
        v[2 * gi + 1] = x[j1];
        nibs |= nib << (4 * gi);
        if (mask) {
#pragma unroll
          for (int p = 0; p < M; ++p) msk[gi][p] = 0;
          msk[gi][(cs >> (8 * j0)) & 0xFF] = 1;
          msk[gi][(cs >> (8 * j1)) & 0xFF] = 1;
        }
      } else {
        v[2 * gi] = (T)0;
        v[2 * gi + 1] = (T)0;
      }
    }
    const int64_t gglob = c0 / M + 4 * q;  // first group of this unit, even
    T* vd = values + row * (G * 2) + gglob * 2;
    if (vec_out && gq == 4) {
      if constexpr (sizeof(T) == 2) {
        u32x4 t; __builtin_memcpy(&t, v, 16); *reinterpret_cast<u32x4*>(vd) = t;
      } else {
        u32x4 t0, t1; __builtin_memcpy(&t0, v, 16); __builtin_memcpy(&t1, v + 4, 16);
        reinterpret_cast<u32x4*>(vd)[0] = t0; reinterpret_cast<u32x4*>(vd)[1] = t1;
      }
    } else {
      for (int e = 0; e < 2 * gq; ++e) vd[e] = v[e];
    }
    uint8_t* md = meta + row * meta_row + gglob / 2;
    if (gq > 2 && ((uintptr_t)md & 1) == 0) {
      *reinterpret_cast<uint16_t*>(md) = (uint16_t)(nibs & 0xFFFF);
    } else {
      md[0] = (uint8_t)(nibs & 0xFF);
      if (gq > 2) md[1] = (uint8_t)((nibs >> 8) & 0xFF);
    }
    if (mask) {
      uint8_t* mk = mask + row * ldmask + c0 + 4 * q * M;
      for (int gi = 0; gi < gq; ++gi)
#pragma unroll
        for (int p = 0; p < M; ++p) mk[gi * M + p] = msk[gi][p];
    }
  }
  __syncthreads();   // every thread is done with the tile before the next one is staged
  }
}

// ---------------------------------------------------------------------------
// The tiled path for bf16 with V in {64, 128, 256} and K a multiple of CW = 256, 256, 64 columns:
// one workgroup per tile (V rows x CW columns, 32 KB, or 64 KB for V = 128) and nothing carried
// from tile to tile, so two to four workgroups share a CU and each ends as soon as its stores are
// issued.  The streaming kernel above
// keeps at most two workgroups per CU (its registers hold the next 64 KB tile) and, walking
// several tiles, waits for each tile's stores before the next one's loads are used; with small
// independent tiles the CU's resident workgroups sit in different phases (loads, column sums,
// selection) and HBM stays busy.  Same rule, same order of the fp64 additions, same outputs.
// Tiles are dealt so that the consecutive column tiles of a V-row block share an XCD, whose L2
// then merges the partial lines of the values and metadata rows they write.
// ---------------------------------------------------------------------------
// Columns of a tile: 256 for V = 128 (a row's 64 values fill a 128-byte line; 66.6 against 69.9 us
// with 128 columns at 8192 x 16384), 16384 / V otherwise.
constexpr int tile_cols(int V) { return V == 128 ? 256 : 16384 / V; }

template <int V, int M, bool RELU>
__global__ __launch_bounds__(256) void venom_prune_tile_kernel(const uint16_t* __restrict__ Z, int64_t ldz,
                                                               int64_t K, uint16_t* __restrict__ values,
                                                               uint8_t* __restrict__ meta,
                                                               uint8_t* __restrict__ colsel, int ntx) {
  constexpr int CW = tile_cols(V);       // columns of a tile
  constexpr int NG = CW / M, NQ = NG / 4;  // groups, quads of groups per tile row
  constexpr int PITCH = CW + 8;          // LDS row pitch in elements (16 bytes of padding)
  constexpr int CPR = CW / 8;            // 16-byte chunks per tile row
  constexpr int NU = V * CPR / 256;      // chunks per thread
  static_assert(NQ >= 1 && (V * CPR) % 256 == 0 && 256 % NQ == 0 && CW <= 256, "tile shape");
  __shared__ __align__(16) uint16_t tile[V * PITCH];
  __shared__ double l1[CW];
  __shared__ uint32_t csel[NG];

  const int tid = threadIdx.x;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t blk = t / ntx, c0 = (int64_t)(t - blk * ntx) * CW;
  const int64_t G = K / M;

  // 1. the tile, ReLU applied, into LDS (16-byte loads, a row's chunks on consecutive lanes)
  u32x4 x[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = tid + 256 * u, r = i / CPR, c = (i % CPR) * 8;
    x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Z + (blk * V + r) * ldz + c0 + c));
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = tid + 256 * u, r = i / CPR, c = (i % CPR) * 8;
    u32x4 v = x[u];
    if constexpr (RELU) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = v[w] & 0xFFFFu, hi = v[w] >> 16;
        v[w] = (Elem<uint16_t>::positive((uint16_t)lo) ? lo : 0u) | ((Elem<uint16_t>::positive((uint16_t)hi) ? hi : 0u) << 16);
      }
    }
    *reinterpret_cast<u32x4*>(tile + r * PITCH + c) = v;
  }
  __syncthreads();

  // 2. column L1 norms in fp64, rows in ascending order (one lane per column)
  if (tid < CW) {
    double a = 0.0;
#pragma unroll 8
    for (int r = 0; r < V; ++r) a += (double)__uint_as_float((uint32_t)(tile[r * PITCH + tid] & 0x7FFFu) << 16);
    l1[tid] = a;
  }
  __syncthreads();

  // 3. per group the 4 columns of largest L1 (lower column on ties): one lane per (group, column),
  //    the group's kept positions packed in ascending order from the wave's ballot
  if (tid < CW) {
    const int g = tid / M, p = tid % M;
    const double kp = l1[tid];
    int rk = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const double kq = l1[g * M + q];
      rk += (kq > kp || (q < p && kq == kp)) ? 1 : 0;
    }
    const uint64_t kept = __ballot(rk < 4);
    if (p == 0) {
      uint32_t rest = (uint32_t)(kept >> ((tid & 63) & ~(M - 1))) & ((1u << M) - 1u), packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        packed |= (uint32_t)__builtin_ctz(rest) << (8 * j);
        rest &= rest - 1u;
      }
      csel[g] = packed;
      *reinterpret_cast<uint32_t*>(colsel + (blk * G + c0 / M + g) * 4) = packed;
    }
  }
  __syncthreads();

  // 4. per (row, quad of groups): 2 of each group's 4 chosen columns by magnitude (lower on ties);
  //    16 bytes of values and 2 bytes of nibbles
  const int q = tid % NQ;
  int ofs[4][4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const uint32_t cs = csel[4 * q + gi];
#pragma unroll
    for (int j = 0; j < 4; ++j) ofs[gi][j] = (4 * q + gi) * M + (int)((cs >> (8 * j)) & 0xFF);
  }
  const int64_t gq = c0 / M + 4 * q;   // the quad's first group, even
  const int64_t meta_row = (G + 1) / 2;
#pragma unroll
  for (int r = tid / NQ; r < V; r += 256 / NQ) {
    const uint16_t* trow = tile + r * PITCH;
    uint32_t out[4], nibs = 0;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = trow[ofs[gi][j]];
      const uint32_t nib = select24_bf16(v[0], v[1], v[2], v[3]);
      const uint32_t d01 = v[0] | (v[1] << 16), d23 = v[2] | (v[3] << 16);
      const uint32_t j0 = nib & 3, j1 = nib >> 2;
      out[gi] = __builtin_amdgcn_perm(d23, d01, (j0 * 0x202u + 0x100u) | ((j1 * 0x202u + 0x100u) << 16));
      nibs |= nib << (4 * gi);
    }
    const int64_t row = blk * V + r;
    *reinterpret_cast<u32x4*>(values + row * (G * 2) + gq * 2) = u32x4{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<uint16_t*>(meta + row * meta_row + gq / 2) = (uint16_t)nibs;
  }
}

// Conditions of the tiled path (the caller has checked R % V == 0 and K % M == 0).
static bool venom_tile_ok(const void* Z, int64_t ldz, int64_t K, int V, const void* values, const uint8_t* meta,
                          const uint8_t* colsel, const uint8_t* mask) {
  if (mask || (V != 64 && V != 128 && V != 256) || env_is_one("NMSPARSE_VENOM_STREAM")) return false;
  const int CW = tile_cols(V);
  return K % CW == 0 && (uintptr_t)Z % 16 == 0 && ldz % 8 == 0 && (uintptr_t)values % 16 == 0 &&
         (uintptr_t)meta % 2 == 0 && (uintptr_t)colsel % 4 == 0;
}

template <int V, int M>
static hipError_t venom_tile_launch(const void* Z, int64_t ldz, int64_t R, int64_t K, int relu, void* values,
                                    uint8_t* meta, uint8_t* colsel, hipStream_t s) {
  const int64_t ntx = K / tile_cols(V), ntiles = (R / V) * ntx;
  if (ntiles > INT32_MAX || ntx > INT32_MAX) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(256), 0, s, (const uint16_t*)Z, ldz, K, (uint16_t*)values,
                       meta, colsel, (int)ntx);
    return hipGetLastError();
  };
  return relu ? go(venom_prune_tile_kernel<V, M, true>) : go(venom_prune_tile_kernel<V, M, false>);
}

template <int V>
static hipError_t venom_tile_dispatch(int M, const void* Z, int64_t ldz, int64_t R, int64_t K, int relu, void* values,
                                      uint8_t* meta, uint8_t* colsel, hipStream_t s) {
  switch (M) {
    case 4: return venom_tile_launch<V, 4>(Z, ldz, R, K, relu, values, meta, colsel, s);
    case 8: return venom_tile_launch<V, 8>(Z, ldz, R, K, relu, values, meta, colsel, s);
    default: return venom_tile_launch<V, 16>(Z, ldz, R, K, relu, values, meta, colsel, s);
  }
}

template <typename T>
static hipError_t venom_dispatch(const void* Z, int64_t ldz, int64_t R, int64_t K, int V, int M, int relu,
                                 void* values, uint8_t* meta, uint8_t* colsel, uint8_t* mask, int64_t ldmask,
                                 hipStream_t s) {
  if (sizeof(T) == 2 && venom_tile_ok(Z, ldz, K, V, values, meta, colsel, mask)) {
    return V == 64    ? venom_tile_dispatch<64>(M, Z, ldz, R, K, relu, values, meta, colsel, s)
           : V == 128 ? venom_tile_dispatch<128>(M, Z, ldz, R, K, relu, values, meta, colsel, s)
                      : venom_tile_dispatch<256>(M, Z, ldz, R, K, relu, values, meta, colsel, s);
  }
  const int esz = sizeof(T);
  int CW = (int)(65536 / ((int64_t)V * esz));
  CW = (CW / 64) * 64;
  if (CW > 512) CW = 512;
  if (CW < 64) CW = 64;
  const size_t lds = (size_t)V * (CW + 8) * esz + (size_t)CW * sizeof(double) + (size_t)(CW / 4) * 4 + 64;
  const int vec_in = ((uintptr_t)Z % 16 == 0) && ((ldz * esz) % 16 == 0);
  const int vec_out = ((uintptr_t)values % 16 == 0) && (((K / M) * 2 * esz) % 16 == 0);
  const int ntx = (int)((K + CW - 1) / CW);
  const int64_t ntiles = (R / V) * (int64_t)ntx;
  const int stream = vec_in && K % CW == 0 && (int64_t)V * (CW / (16 / esz)) == 256 * kStreamChunks;
  // streaming path: two resident workgroups per CU walk the tiles; otherwise one workgroup per tile
  const int64_t grid = stream ? (ntiles < 512 ? ntiles : 512) : ntiles;
  auto run = [&](auto kern) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, (const T*)Z, ldz, K, V, relu, CW, (T*)values,
                       meta, colsel, mask, ldmask, vec_in, vec_out, ntx, ntiles, stream);
    return hipGetLastError();
  };
  switch (M) {
    case 4: return run(venom_prune_kernel<T, 4>);
    case 8: return run(venom_prune_kernel<T, 8>);
    default: return run(venom_prune_kernel<T, 16>);
  }
}

hipError_t launch_prune_act_venom(int dt, const void* Z, int64_t ldz, int64_t R, int64_t K, int V, int M,
                                  int relu, void* values, uint8_t* meta, uint8_t* colsel, uint8_t* mask,
                                  int64_t ldmask, hipStream_t s) {
  return dt == DT_BF16
             ? venom_dispatch<uint16_t>(Z, ldz, R, K, V, M, relu, values, meta, colsel, mask, ldmask, s)
             : venom_dispatch<uint32_t>(Z, ldz, R, K, V, M, relu, values, meta, colsel, mask, ldmask, s);
}

}  // namespace nms
