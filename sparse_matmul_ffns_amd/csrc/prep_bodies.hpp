// Bodies of the streaming kernels that a fused launch also runs (workgroups of 256 threads;
// `bid` is the workgroup's index within the kernel's own grid).
#pragma once

#include "common.hpp"

namespace nms {

// ---------------------------------------------------------------------------
// nm_prune_compress, 2:4 with 16-byte aligned rows: the selection of nm_prune and the packing of
// nm_compress in one pass over A (one read of A instead of two, no read of the mask).  One thread
// per 16 elements (4 groups) and kFusedU such chunks, all loaded before any is ranked: 16-byte
// loads of A, one 16-byte store of the chunk's mask bytes, one 16- or 32-byte store of its 8 kept
// values and one 2-byte store of its 4 nibbles.  Values and metadata are written with ordinary
// stores (the SpMM reads them next and finds them in the last-level cache); the mask, which
// nothing in the step reads, with non-temporal ones.  I is the chunk index type, U the chunks per
// thread: kFusedU for the prune kernel alone, kPrepU inside the fused prep launch, where smaller
// workgroups (twice as many) finish the launch sooner (18.7 against 19.5 us at A [8192 x 2048],
// B [2048 x 4096]).
// ---------------------------------------------------------------------------
constexpr int kFusedU = 2;
constexpr int kPrepU = 1;

template <typename T, typename I, int U = kFusedU>
__device__ __forceinline__ void prune_compress24_body(int bid, const T* __restrict__ A, int64_t lda, int64_t R,
                                                      int64_t K, uint8_t* __restrict__ mask, int64_t ldmask,
                                                      T* __restrict__ values, uint8_t* __restrict__ meta) {
  constexpr int NA = (int)sizeof(T);               // 16-byte loads of A per chunk (16 elements)
  const I per_row = (I)(K / 16);
  const I total = (I)R * per_row;
  const I base = (I)bid * (256 * U) + threadIdx.x;
  u32x4 xa[U][NA];
  I rr[U], cc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const I cid = base + 256 * u;
    rr[u] = cid / per_row;
    cc[u] = (cid - rr[u] * per_row) * 16;
    if (cid < total) {
      const u32x4* a4 = reinterpret_cast<const u32x4*>(A + (int64_t)rr[u] * lda + cc[u]);
#pragma unroll
      for (int q = 0; q < NA; ++q) xa[u][q] = __builtin_nontemporal_load(a4 + q);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (base + 256 * u >= total) break;
    const int64_t r = rr[u], c0 = cc[u];
    uint32_t out[2 * NA];   // the 8 kept values of the chunk, packed
    uint32_t mk[4];         // mask bytes of the 4 groups
    uint32_t nibs = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t nib;
      if constexpr (sizeof(T) == 2) {
        const uint32_t d01 = xa[u][g >> 1][(g & 1) * 2], d23 = xa[u][g >> 1][(g & 1) * 2 + 1];
        nib = select24_bf16(d01 & 0xFFFFu, d01 >> 16, d23 & 0xFFFFu, d23 >> 16);
        const uint32_t p0 = nib & 3u, p1 = nib >> 2;
        // bytes 2p, 2p+1 of the pair (d23:d01) hold the group's value p
        out[g] = __builtin_amdgcn_perm(d23, d01, (p0 * 0x202u + 0x100u) | ((p1 * 0x202u + 0x100u) << 16));
      } else {
        const u32x4 q = xa[u][g];
        nib = select24(q[0] & 0x7FFFFFFFu, q[1] & 0x7FFFFFFFu, q[2] & 0x7FFFFFFFu, q[3] & 0x7FFFFFFFu);
        const uint32_t p0 = nib & 3u, p1 = nib >> 2;
        auto pick = [&](uint32_t p) { return p == 0 ? q[0] : p == 1 ? q[1] : p == 2 ? q[2] : q[3]; };
        out[2 * g] = pick(p0);
        out[2 * g + 1] = pick(p1);
      }
      mk[g] = (1u << (8 * (nib & 3u))) | (1u << (8 * (nib >> 2)));
      nibs |= nib << (4 * g);
    }
    __builtin_nontemporal_store(u32x4{mk[0], mk[1], mk[2], mk[3]},
                                reinterpret_cast<u32x4*>(mask + r * ldmask + c0));
    T* vd = values + r * (K / 2) + c0 / 2;
#pragma unroll
    for (int q = 0; q < NA / 2; ++q)
      reinterpret_cast<u32x4*>(vd)[q] = u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
    *reinterpret_cast<uint16_t*>(meta + r * (K / 8) + c0 / 8) = (uint16_t)nibs;
  }
}

// ---------------------------------------------------------------------------
// Transpose of a bf16 matrix: dst[c][r] = src[r][c].  A lane moves an 8 x 8
// block: eight 16-byte row loads, v_perm into eight 8-row columns, eight
// 16-byte stores.  The 64 lanes of a wave cover a 64 x 64 tile (lanes 8b..8b+7
// take row block b), so both the loads and the stores of a wave cover whole
// 128-byte runs.  Edges (rows or columns not a multiple of 8) take the
// element-wise path.  The result is written with ordinary stores: the SpMM reads
// it right after, and non-temporal stores (which bypass the last-level cache)
// made that SpMM ~11% slower at 8192 x 2048 x 4096.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose_bf16_body(int bid, const uint16_t* __restrict__ src, int64_t lds, int64_t R,
                                                    int64_t Cn, uint16_t* __restrict__ dst, int64_t ldd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tiles_c = (Cn + 63) / 64;
  const int64_t tile = (int64_t)bid * 4 + wave;
  const int64_t tr = tile / tiles_c, tc = tile % tiles_c;
  const int64_t r0 = tr * 64 + 8 * (lane & 7), c0 = tc * 64 + 8 * (lane >> 3);
  if (r0 >= R || c0 >= Cn) return;
  const bool full = r0 + 8 <= R && c0 + 8 <= Cn && lds % 8 == 0 && ldd % 8 == 0 && (uintptr_t)src % 16 == 0 &&
                    (uintptr_t)dst % 16 == 0;
  if (full) {
    u32x4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (r0 + q) * lds + c0));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = __builtin_amdgcn_perm(v[2 * j + 1][e >> 1], v[2 * j][e >> 1], sel);
      *reinterpret_cast<u32x4*>(dst + (c0 + e) * ldd + r0) = d;
    }
  } else {
    for (int q = 0; q < 8 && r0 + q < R; ++q)
      for (int e = 0; e < 8 && c0 + e < Cn; ++e) dst[(c0 + e) * ldd + r0 + q] = src[(r0 + q) * lds + c0 + e];
  }
}

}  // namespace nms
