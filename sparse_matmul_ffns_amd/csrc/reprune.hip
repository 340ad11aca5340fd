// Double pruning of the transposed weight (gfx950).
//
// The SLOPE abstract (NSF PAR award 2340011) runs the backward pass on the
// transposed weight re-pruned with N:M.  Here the already 2:4-pruned weight
// W_s [R x K] (compressed along K) is decompressed with +0.0 fill, transposed
// and pruned 2:4 along R, giving W_ds^T [K x R] compressed along R.
//
// bf16 operands whose sides are multiples of 128 take the tiled kernel below
// (reprune_t_bf16_kernel); the others this one, where one workgroup owns a
// 128-row x 64-column tile of W_s:
//   1. each lane decompresses 4 groups (16 columns of one row) into LDS;
//   2. each lane takes 16 consecutive rows of one column (4 output groups),
//      keeps 2 of every 4 by magnitude (lower row on ties) and writes 8 values
//      and 2 bytes of nibbles; the 8 lanes of one column write 128 contiguous
//      bytes of the output row.
// HBM traffic is one read of W_s's values and metadata and one write of the
// result, the bound of this pass.
#include "common.hpp"
#include "launch.hpp"
#include "prep_bodies.hpp"

namespace nms {

constexpr int RP_ROWS = 128;  // rows of W_s per tile
constexpr int RP_COLS = 64;   // columns of W_s per tile
constexpr int RP_PITCH = RP_COLS + 2;

template <typename T>
__global__ __launch_bounds__(256) void reprune_t_kernel(const T* __restrict__ values, const uint8_t* __restrict__ meta,
                                                        int64_t R, int64_t K, T* __restrict__ values_t,
                                                        uint8_t* __restrict__ meta_t, int vec_in, int vec_out) {
  __shared__ T tile[RP_ROWS * RP_PITCH];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * RP_ROWS;
  const int64_t k0 = (int64_t)blockIdx.y * RP_COLS;
  const int64_t kvalid = (K - k0) < RP_COLS ? (K - k0) : RP_COLS;   // multiple of 4
  const int64_t rvalid = (R - r0) < RP_ROWS ? (R - r0) : RP_ROWS;   // multiple of 4

  // 1. decompress: unit = (row, quad of 4 groups); 128 rows x 4 quads
  for (int u = tid; u < RP_ROWS * 4; u += 256) {
    const int r = u >> 2, q = u & 3;
    const int c = q * 16;
    T dense[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) dense[e] = (T)0;
    if (r < rvalid && c < kvalid) {
      const int64_t row = r0 + r;
      const T* v = values + row * (K / 2) + (k0 + c) / 2;
      const uint8_t* m = meta + row * ((K + 7) / 8) + (k0 + c) / 8;
      const int ng = (int)((kvalid - c) < 16 ? (kvalid - c) : 16) / 4;
      T vv[8];
      uint32_t nibs = 0;
      if (vec_in && ng == 4) {
        if constexpr (sizeof(T) == 2) {
          u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v));
          __builtin_memcpy(vv, &t, 16);
        } else {
          u32x4 t0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v));
          u32x4 t1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v) + 1);
          __builtin_memcpy(vv, &t0, 16);
          __builtin_memcpy(vv + 4, &t1, 16);
        }
        nibs = (uint32_t)m[0] | ((uint32_t)m[1] << 8);
      } else {
        // groups of this unit start at column k0 + c; the first one may sit in
        // the high nibble when (k0 + c) / 4 is odd (never here: c and k0 are
        // multiples of 16)
        for (int g = 0; g < ng; ++g) {
          vv[2 * g] = v[2 * g];
          vv[2 * g + 1] = v[2 * g + 1];
          nibs |= (uint32_t)((m[g >> 1] >> (4 * (g & 1))) & 0xF) << (4 * g);
        }
      }
      for (int g = 0; g < ng; ++g) {
        const uint32_t nib = (nibs >> (4 * g)) & 0xF;
        dense[4 * g + (nib & 3)] = vv[2 * g];
        dense[4 * g + ((nib >> 2) & 3)] = vv[2 * g + 1];
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[r * RP_PITCH + c + e] = dense[e];
  }
  __syncthreads();

  // 2. re-prune along rows: unit = (column, 16-row chunk); chunk index fastest
  for (int u = tid; u < RP_COLS * 8; u += 256) {
    const int col = u >> 3, ch = u & 7;
    const int rr = ch * 16;
    if (col >= kvalid || rr >= rvalid) continue;
    const int ng = (int)((rvalid - rr) < 16 ? (rvalid - rr) : 16) / 4;
    T out[8];
    uint32_t nibs = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T x[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) x[p] = tile[(rr + 4 * g + p) * RP_PITCH + col];
      const uint32_t nib = select24(Elem<T>::key(x[0]), Elem<T>::key(x[1]), Elem<T>::key(x[2]), Elem<T>::key(x[3]));
      out[2 * g] = x[nib & 3];
      out[2 * g + 1] = x[(nib >> 2) & 3];
      nibs |= nib << (4 * g);
    }
    const int64_t orow = k0 + col;
    T* vd = values_t + orow * (R / 2) + (r0 + rr) / 2;
    uint8_t* md = meta_t + orow * ((R + 7) / 8) + (r0 + rr) / 8;
    if (vec_out && ng == 4) {
      if constexpr (sizeof(T) == 2) {
        u32x4 t; __builtin_memcpy(&t, out, 16); *reinterpret_cast<u32x4*>(vd) = t;
      } else {
        u32x4 t0, t1; __builtin_memcpy(&t0, out, 16); __builtin_memcpy(&t1, out + 4, 16);
        reinterpret_cast<u32x4*>(vd)[0] = t0; reinterpret_cast<u32x4*>(vd)[1] = t1;
      }
      md[0] = (uint8_t)(nibs & 0xFF);
      md[1] = (uint8_t)(nibs >> 8);
    } else {
      for (int e = 0; e < 2 * ng; ++e) vd[e] = out[e];
      // (r0 + rr) / 4 is even, so group g of this unit is nibble g of md
      for (int g = 0; g < ng; g += 2) {
        const uint32_t lo = (nibs >> (4 * g)) & 0xF;
        const uint32_t hi = (g + 1 < ng) ? ((nibs >> (4 * (g + 1))) & 0xF) : 0u;
        md[g >> 1] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

// bf16 tiles of 128 rows x 128 columns of W_s, whole 128-byte lines in and out.
//   1. Unit (row r, 16-column chunk c): lane l of a wave takes chunk l%8 of row l/8 + 8i, so each
//      load instruction reads 8 whole 128-byte rows of values; the four units of a lane are
//      loaded one tile ahead, while the workgroup works on the previous tile.  The 16 dense
//      columns are written to LDS as two 16-byte runs; the LDS row holds the 128 columns as 64
//      dwords, run c of row r at dword 8(c ^ s(r)), s(r) = (r / 16) % 8.
//   2. Unit (column pair j, 16-row chunk ch), chunk fastest: 16 dword reads give both columns of
//      16 rows (the lanes of one read hit 64 distinct banks through the XOR); each column's 4
//      groups of 4 rows keep their 2 largest magnitudes; the 8 lanes of a pair write 128
//      contiguous bytes of each of the two output rows.
constexpr int RB_TILE = 128;

// Tiles t = first, first + stride, ... of the re-prune (the kernel below runs one per workgroup;
// the fused launch with a transpose passes its own numbering).  PANELS: the output in the panel
// layout of spmm_nm_t_panels (R a multiple of 256; the same values and nibbles, each 16-byte
// values piece and 2-byte metadata piece at its panel address).
template <bool PANELS = false>
__device__ __forceinline__ void reprune_t_bf16_body(uint32_t first, uint32_t stride, uint32_t* __restrict__ tile,
                                                    const uint16_t* __restrict__ values,
                                                    const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                    uint16_t* __restrict__ values_t, uint8_t* __restrict__ meta_t) {
  const int tid = threadIdx.x;
  const int64_t vrow = K / 2, mrow = K / 8;
  const uint32_t nbx = (uint32_t)(R / RB_TILE), ntiles = nbx * (uint32_t)(K / RB_TILE);

  // a workgroup walks tiles t, t + gridDim.x, ...; the next tile's loads are in flight while the
  // current one is re-pruned and written
  u32x4 v[4];
  uint32_t m[4];
  // tile t -> logical tile L: each XCD (workgroups t % 8) takes a contiguous range of logical
  // tiles, so the 8 neighbouring tiles whose 16-byte metadata runs share one 128-byte output
  // line are written through one L2
  const bool remap = ntiles % 8 == 0;
  auto logical = [&](uint32_t t) { return remap ? (t % 8) * (ntiles / 8) + t / 8 : t; };
  auto load = [&](uint32_t t) {
    t = logical(t);
    const int64_t r0 = (int64_t)(t % nbx) * RB_TILE, k0 = (int64_t)(t / nbx) * RB_TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int64_t row = r0 + (u >> 3);
      const int c = u & 7;
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(values + row * vrow + k0 / 2 + 8 * c));
      m[i] = *reinterpret_cast<const uint16_t*>(meta + row * mrow + k0 / 8 + 2 * c);
    }
  };
  if (first < ntiles) load(first);
  for (uint32_t t = first; t < ntiles; t += stride) {
    const uint32_t lt = logical(t);
    const int64_t r0 = (int64_t)(lt % nbx) * RB_TILE, k0 = (int64_t)(lt / nbx) * RB_TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 3, c = u & 7;
      uint32_t d[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t nib = (m[i] >> (4 * g)) & 0xF;
        const uint32_t p0 = nib & 3, p1 = nib >> 2;
        const uint32_t a = v[i][g] & 0xFFFF, b = v[i][g] >> 16;
        uint32_t x[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) x[p] = (p == (int)p1) ? b : ((p == (int)p0) ? a : 0u);
        d[2 * g] = x[0] | (x[1] << 16);
        d[2 * g + 1] = x[2] | (x[3] << 16);
      }
      // odd rows write their second 16-byte half first: the 16 lanes of two rows then cover all
      // 64 banks in each write
      uint32_t* dst = tile + r * 64 + 8 * (c ^ ((r >> 4) & 7));
      const bool odd = r & 1;
      *reinterpret_cast<u32x4*>(dst + (odd ? 4 : 0)) =
          odd ? u32x4{d[4], d[5], d[6], d[7]} : u32x4{d[0], d[1], d[2], d[3]};
      *reinterpret_cast<u32x4*>(dst + (odd ? 0 : 4)) =
          odd ? u32x4{d[0], d[1], d[2], d[3]} : u32x4{d[4], d[5], d[6], d[7]};
    }
    if (t + stride < ntiles) load(t + stride);
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      const int ch = u & 7, j = u >> 3;
      uint32_t x[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = tile[(16 * ch + e) * 64 + (j ^ (8 * ch))];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // the column's 16-bit halves of rows 4h..4h+3 packed as (d23:d01); value q is bytes 2q, 2q+1
        const uint32_t pick = half ? 0x07060302u : 0x05040100u;
        uint32_t out[4];
        uint32_t nibs = 0;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t d01 = __builtin_amdgcn_perm(x[4 * h + 1], x[4 * h], pick);
          const uint32_t d23 = __builtin_amdgcn_perm(x[4 * h + 3], x[4 * h + 2], pick);
          const uint32_t nib = select24(Elem<uint16_t>::key((uint16_t)(d01 & 0xFFFF)),
                                        Elem<uint16_t>::key((uint16_t)(d01 >> 16)),
                                        Elem<uint16_t>::key((uint16_t)(d23 & 0xFFFF)),
                                        Elem<uint16_t>::key((uint16_t)(d23 >> 16)));
          const uint32_t q0 = nib & 3, q1 = nib >> 2;
          out[h] = __builtin_amdgcn_perm(d23, d01, (q0 * 0x202u + 0x100u) | ((q1 * 0x202u + 0x100u) << 16));
          nibs |= nib << (4 * h);
        }
        const int64_t orow = k0 + 2 * j + half, oc = r0 + 16 * ch;   // output row, its dense column
        uint16_t* vd;
        uint8_t* md;
        if constexpr (PANELS) {
          vd = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(values_t) +
                                           ((orow >> 1) * (R / 64) + oc / 64) * 128 + (orow & 1) * 64 + oc % 64);
          md = meta_t + ((orow >> 2) * (R / 256) + oc / 256) * 128 + (orow & 3) * 32 + (oc % 256) / 8;
        } else {
          vd = values_t + orow * (R / 2) + oc / 2;
          md = meta_t + orow * (R / 8) + oc / 8;
        }
        *reinterpret_cast<u32x4*>(vd) = u32x4{out[0], out[1], out[2], out[3]};
        *reinterpret_cast<uint16_t*>(md) = (uint16_t)nibs;
      }
    }
    __syncthreads();   // every lane is done with the tile before the next one is written
  }
}

__global__ __launch_bounds__(256) void reprune_t_bf16_kernel(const uint16_t* __restrict__ values,
                                                             const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                             uint16_t* __restrict__ values_t,
                                                             uint8_t* __restrict__ meta_t) {
  __shared__ uint32_t tile[RB_TILE * 64];
  reprune_t_bf16_body(blockIdx.x, gridDim.x, tile, values, meta, R, K, values_t, meta_t);
}

// The re-prune of a training step's weight and the transpose of its input in one launch (they
// touch disjoint data, and each alone spends part of its time filling and draining the chip):
// one re-prune tile per workgroup first, the transpose's workgroups after them, each running
// exactly the code of its own kernel.  The transpose goes last, as in the two-launch order, so
// X^T is the freshest data in the last-level cache when the forward product reads it; with the
// transpose first, the step's later products measured ~5 us slower at d_model 4096, d_ff 16384,
// 8192 tokens.
template <bool PANELS>
__global__ __launch_bounds__(256) void reprune_transpose_kernel(const uint16_t* __restrict__ values,
                                                                const uint8_t* __restrict__ meta, int64_t R,
                                                                int64_t K, uint16_t* __restrict__ values_t,
                                                                uint8_t* __restrict__ meta_t,
                                                                const uint16_t* __restrict__ X, int64_t ldx,
                                                                int64_t RX, int64_t CX, uint16_t* __restrict__ Xt,
                                                                int64_t ldxt, uint32_t n_reprune) {
  __shared__ uint32_t tile[RB_TILE * 64];
  const int b = blockIdx.x;
  if (b < (int)n_reprune)
    reprune_t_bf16_body<PANELS>((uint32_t)b, n_reprune, tile, values, meta, R, K, values_t, meta_t);
  else
    transpose_bf16_body(b - (int)n_reprune, X, ldx, RX, CX, Xt, ldxt);
}

template <typename T>
static hipError_t reprune_dispatch(const void* values, const uint8_t* meta, int64_t R, int64_t K, void* values_t,
                                   uint8_t* meta_t, hipStream_t s) {
  const int esz = sizeof(T);
  if (esz == 2 && R % RB_TILE == 0 && K % RB_TILE == 0 && (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 2 == 0 &&
      (uintptr_t)values_t % 16 == 0 && (uintptr_t)meta_t % 2 == 0 && !force_generic()) {
    // one workgroup per tile (measured: 35.6 us against 37.6 with 1024 workgroups walking four
    // tiles each at 16384 x 4096, 31.9 against 36.2 at 4096 x 16384); the walk only serves grids
    // past 2^30 tiles
    const int64_t ntiles = (R / RB_TILE) * (K / RB_TILE);
    const unsigned grid = (unsigned)(ntiles < (int64_t(1) << 30) ? ntiles : (int64_t(1) << 30));
    hipLaunchKernelGGL(reprune_t_bf16_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)values, meta, R, K,
                       (uint16_t*)values_t, meta_t);
    return hipGetLastError();
  }
  const int vec_in = ((uintptr_t)values % 16 == 0) && (((K / 2) * esz) % 16 == 0);
  const int vec_out = ((uintptr_t)values_t % 16 == 0) && (((R / 2) * esz) % 16 == 0);
  dim3 grid((unsigned)((R + RP_ROWS - 1) / RP_ROWS), (unsigned)((K + RP_COLS - 1) / RP_COLS));
  hipLaunchKernelGGL(reprune_t_kernel<T>, grid, dim3(256), 0, s, (const T*)values, meta, R, K, (T*)values_t, meta_t,
                     vec_in, vec_out);
  return hipGetLastError();
}

hipError_t launch_nm_reprune_t(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                               void* values_t, uint8_t* meta_t, hipStream_t s) {
  return dt == DT_BF16 ? reprune_dispatch<uint16_t>(values, meta, R, K, values_t, meta_t, s)
                       : reprune_dispatch<uint32_t>(values, meta, R, K, values_t, meta_t, s);
}

hipError_t launch_nm_reprune_t_transpose(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                         void* values_t, uint8_t* meta_t, const void* X, int64_t ldx, int64_t RX,
                                         int64_t CX, void* Xt, int64_t ldxt, hipStream_t s) {
  const bool fused = dt == DT_BF16 && R % RB_TILE == 0 && K % RB_TILE == 0 && (uintptr_t)values % 16 == 0 &&
                     (uintptr_t)meta % 2 == 0 && (uintptr_t)values_t % 16 == 0 && (uintptr_t)meta_t % 2 == 0 &&
                     !force_generic();
  const int64_t n_reprune = (R / RB_TILE) * (K / RB_TILE);
  const int64_t tiles = ((RX + 63) / 64) * ((CX + 63) / 64);
  const int64_t n_transpose = (tiles + 3) / 4;
  if (!fused || n_reprune + n_transpose > (int64_t)INT32_MAX) {   // the two calls, each with its own paths
    const hipError_t e = launch_nm_reprune_t(dt, values, meta, R, K, values_t, meta_t, s);
    if (e != hipSuccess) return e;
    return launch_nm_transpose(dt, X, ldx, RX, CX, Xt, ldxt, s);
  }
  hipLaunchKernelGGL(reprune_transpose_kernel<false>, dim3((unsigned)(n_reprune + n_transpose)), dim3(256), 0, s,
                     (const uint16_t*)values, meta, R, K, (uint16_t*)values_t, meta_t, (const uint16_t*)X, ldx, RX, CX,
                     (uint16_t*)Xt, ldxt, (uint32_t)n_reprune);
  return hipGetLastError();
}

// The same launch with the re-pruned transpose in the panel layout: bf16, R a multiple of 256 and
// K of 128, the aligned layout of the tiled re-prune; no fallback.
hipError_t launch_nm_reprune_t_transpose_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                                void* values_t, uint8_t* meta_t, const void* X, int64_t ldx,
                                                int64_t RX, int64_t CX, void* Xt, int64_t ldxt, hipStream_t s) {
  if (R % 256 != 0 || K % RB_TILE != 0 || (uintptr_t)values % 16 != 0 || (uintptr_t)meta % 2 != 0 ||
      (uintptr_t)values_t % 16 != 0 || (uintptr_t)meta_t % 2 != 0)
    return hipErrorNotSupported;
  const int64_t n_reprune = (R / RB_TILE) * (K / RB_TILE);
  const int64_t tiles = ((RX + 63) / 64) * ((CX + 63) / 64);
  const int64_t n_transpose = (tiles + 3) / 4;
  if (n_reprune + n_transpose > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reprune_transpose_kernel<true>, dim3((unsigned)(n_reprune + n_transpose)), dim3(256), 0, s,
                     (const uint16_t*)values, meta, R, K, (uint16_t*)values_t, meta_t, (const uint16_t*)X, ldx, RX, CX,
                     (uint16_t*)Xt, ldxt, (uint32_t)n_reprune);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-major 2:4 form -> panel layout (spmm_nm_t_panels): one thread per 16-byte piece of the
// output, values first, then metadata; R a multiple of 4, K of 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nm_to_panels_kernel(const uint8_t* __restrict__ values,
                                                           const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                           uint8_t* __restrict__ values_p, uint8_t* __restrict__ meta_p) {
  const int64_t nv = R * K / 16, nm = R * K / 128;   // 16-byte pieces of values (R x K bytes) and metadata
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nv) {
    const int64_t KT = K / 64, L = i / 8, w = (i % 8) * 16;   // line (row pair, step), byte in the line
    const int64_t r = 2 * (L / KT) + w / 64, st = L % KT;
    *reinterpret_cast<u32x4*>(values_p + 16 * i) =
        *reinterpret_cast<const u32x4*>(values + r * K + st * 64 + w % 64);
  } else if (i < nv + nm) {
    const int64_t j = i - nv, KC = K / 256, L = j / 8, w = (j % 8) * 16;   // line (4 rows, chunk)
    const int64_t r = 4 * (L / KC) + w / 32, c = L % KC;
    *reinterpret_cast<u32x4*>(meta_p + 16 * j) = *reinterpret_cast<const u32x4*>(meta + r * (K / 8) + c * 32 + w % 32);
  }
}

hipError_t launch_nm_to_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K, void* values_p,
                               uint8_t* meta_p, hipStream_t s) {
  if (R % 4 != 0 || K % 256 != 0 || (uintptr_t)values % 16 != 0 || (uintptr_t)meta % 16 != 0 ||
      (uintptr_t)values_p % 16 != 0 || (uintptr_t)meta_p % 16 != 0)
    return hipErrorNotSupported;
  const int64_t n = R * K / 16 + R * K / 128;
  if ((n + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(nm_to_panels_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const uint8_t*)values,
                     meta, R, K, (uint8_t*)values_p, meta_p);
  return hipGetLastError();
}

}  // namespace nms
