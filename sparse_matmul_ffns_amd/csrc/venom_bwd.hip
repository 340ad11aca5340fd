// Backward of a down-projection whose input activations are V:N:M sparse (gfx950).
//
// Forward ("To 2:4 Sparsity and Beyond", abstract: v:n:m activations in every FFN matmul; ReLU
// activations as in "Sparser, Faster, Lighter Transformer Language Models", Methodologie):
//   Y [T][Nc] = h_s [T][F] . W_down [F][Nc],  h_s the V:N:M form of h = ReLU(z) (V-blocks of
//   tokens, groups of M along F; values / nibbles / colsel as prune_act_venom writes them).
// Backward products:
//   dZ[t][2g+s] = (dY . W_down^T)[t][g*M + colsel[t/V][g][j_s]]  x  [h_s value > 0] (with ReLU)
//       -- only the kept activations carry a gradient (sddmm_venom: the pipelined SDDMM with the
//          B rows gathered through colsel, sddmm.hip; a SIMT kernel below otherwise);
//   dW_down[k][c] = sum_t h_s[t][k] dY[t][c]
//       -- the reduction runs over tokens, and every V-block of tokens selects a different half of
//          each group's rows, so no 32-row fragment of the product is empty in any block: the
//          matrix instructions cannot skip work.  The fast path writes h_s^T densely
//          (venom_expand_t_kernel, into caller work memory) and runs the dense NT GEMM of
//          sddmm.hip on (h^T, dY^T); a SIMT kernel reads the compressed form directly otherwise.
#include "common.hpp"
#include "launch.hpp"

namespace nms {

// Kept column j_s of (t, g): nibble of h_meta, index into the V-block's colsel entry.
__device__ inline int vnm_kept_col(const uint8_t* meta, const uint8_t* colsel, int64_t t, int64_t g, int s, int V,
                                   int M, int64_t G) {
  const uint32_t nib = (meta[t * ((G + 1) / 2) + g / 2] >> (4 * (g & 1))) & 0xF;
  const uint32_t j = s ? (nib >> 2) & 3 : nib & 3;
  return (int)(g * M + (colsel[((t / V) * G + g) * 4 + j] & (M - 1)));
}

// SIMT dZ: one thread per (token, group), both kept entries; plain fp32 dot products.
template <typename T>
__global__ __launch_bounds__(256) void sddmm_venom_generic_kernel(
    const T* __restrict__ dY, int64_t lddy, const T* __restrict__ Wd, int64_t ldw, int64_t Tn, int64_t F,
    int64_t Nc, int V, int M, const T* __restrict__ hv, const uint8_t* __restrict__ hm,
    const uint8_t* __restrict__ hc, int relu, float* __restrict__ dz) {
  const int64_t G = F / M;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= Tn * G) return;
  const int64_t t = u / G, g = u % G;
  const int c0 = vnm_kept_col(hm, hc, t, g, 0, V, M, G), c1 = vnm_kept_col(hm, hc, t, g, 1, V, M, G);
  float a0 = 0.f, a1 = 0.f;
  for (int64_t c = 0; c < Nc; ++c) {
    const float y = Elem<T>::to_f32(dY[t * lddy + c]);
    a0 = fmaf(y, Elem<T>::to_f32(Wd[c0 * ldw + c]), a0);
    a1 = fmaf(y, Elem<T>::to_f32(Wd[c1 * ldw + c]), a1);
  }
  if (relu) {
    if (!Elem<T>::positive(hv[t * 2 * G + 2 * g])) a0 = 0.f;
    if (!Elem<T>::positive(hv[t * 2 * G + 2 * g + 1])) a1 = 0.f;
  }
  dz[t * 2 * G + 2 * g] = a0;
  dz[t * 2 * G + 2 * g + 1] = a1;
}

// SIMT dW_down: one thread per output (k, c); tokens in order, the kept value looked up from the
// compressed form (0 where token t does not keep column k).
template <typename T>
__global__ __launch_bounds__(256) void spmm_venom_tn_generic_kernel(
    const T* __restrict__ hv, const uint8_t* __restrict__ hm, const uint8_t* __restrict__ hc, int64_t Tn, int64_t F,
    int V, int M, const T* __restrict__ dYt, int64_t lddyt, int64_t Nc, float* __restrict__ dW, int64_t lddw) {
  const int64_t G = F / M;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= F * Nc) return;
  const int64_t k = u / Nc, c = u % Nc, g = k / M;
  const uint32_t p = (uint32_t)(k % M);
  float acc = 0.f;
  for (int64_t t = 0; t < Tn; ++t) {
    const uint32_t sel = *reinterpret_cast<const uint32_t*>(hc + ((t / V) * G + g) * 4);
    const uint32_t nib = (hm[t * ((G + 1) / 2) + g / 2] >> (4 * (g & 1))) & 0xF;
    const uint32_t j0 = nib & 3, j1 = (nib >> 2) & 3;
    int s = -1;
    if (((sel >> (8 * j0)) & (uint32_t)(M - 1)) == p) s = 0;
    else if (((sel >> (8 * j1)) & (uint32_t)(M - 1)) == p) s = 1;
    if (s >= 0) acc = fmaf(Elem<T>::to_f32(hv[t * 2 * G + 2 * g + s]), Elem<T>::to_f32(dYt[c * lddyt + t]), acc);
  }
  dW[k * lddw + c] = acc;
}

// h_s^T written densely: Ht[k][t] = the kept value of (t, k), +0.0 elsewhere.  One workgroup per
// 64 tokens x 128 rows of F: the tile is cleared in LDS, each thread scatters the kept values of
// its (token, group) pairs into it, and the tile leaves as 128-byte row pieces (16-byte stores).
constexpr int XT_T = 64, XT_F = 128;
__global__ __launch_bounds__(256) void venom_expand_t_kernel(const uint16_t* __restrict__ hv,
                                                             const uint8_t* __restrict__ hm,
                                                             const uint8_t* __restrict__ hc, int64_t Tn, int64_t F,
                                                             int V, int M, uint16_t* __restrict__ Ht, int64_t ldh) {
  __shared__ __align__(16) uint16_t tile[XT_F][XT_T + 8];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * XT_T, k0 = (int64_t)blockIdx.y * XT_F;
  const int64_t G = F / M;
  for (int i = tid; i < XT_F * (XT_T + 8) / 8; i += 256)
    reinterpret_cast<u32x4*>(&tile[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  const int gpt = XT_F / M;   // groups in the tile
  for (int u = tid; u < XT_T * gpt; u += 256) {
    const int tl = u / gpt, gl = u % gpt;
    const int64_t t = t0 + tl, g = k0 / M + gl;
    if (t >= Tn || g >= G) continue;
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(hv + t * 2 * G + 2 * g);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int col = vnm_kept_col(hm, hc, t, g, s, V, M, G);
      tile[col - k0][tl] = (uint16_t)(pair >> (16 * s));
    }
  }
  __syncthreads();
  // 128 rows x 128 bytes: 8 lanes per row, 16 bytes each
  for (int i = tid; i < XT_F * 8; i += 256) {
    const int r = i >> 3, piece = i & 7;
    const int64_t k = k0 + r, t = t0 + 8 * piece;
    if (k >= F || t >= Tn) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[r][8 * piece]);
    if (t + 8 <= Tn) {
      *reinterpret_cast<u32x4*>(Ht + k * ldh + t) = v;
    } else {
      for (int q = 0; q < 8 && t + q < Tn; ++q) Ht[k * ldh + t + q] = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
    }
  }
}

// The same with whole-vector loads: a thread takes one token and four consecutive groups, reading
// their kept pairs (16 bytes), nibbles (2 bytes) and column choices (16 bytes) with one load each
// instead of a load per byte.  Tiles of 64 tokens x 128 rows, so a tile's tokens lie in one
// V-block (V % 64 == 0); the LDS row pitch of 72 elements keeps the 16-byte reads of the
// write-out aligned, and the 8-token chunks of row r sit at chunk ^ ((r >> 4) & 7), so the rows a
// wave writes at once (16, 32 or 64 apart) fall on different banks.
template <int M>
__global__ __launch_bounds__(256) void venom_expand_t_vec_kernel(const uint16_t* __restrict__ hv,
                                                                 const uint8_t* __restrict__ hm,
                                                                 const uint8_t* __restrict__ hc, int64_t F, int V,
                                                                 uint16_t* __restrict__ Ht, int64_t ldh) {
  constexpr int NG = XT_F / M, NQ = NG / 4;   // groups and quads of groups of a tile row
  static_assert(NQ >= 1 && 256 % NQ == 0, "tile");
  __shared__ __align__(16) uint16_t tile[XT_F][XT_T + 8];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * XT_T, k0 = (int64_t)blockIdx.y * XT_F;
  const int64_t G = F / M;
  for (int i = tid; i < XT_F * (XT_T + 8) / 8; i += 256)
    reinterpret_cast<u32x4*>(&tile[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  for (int u = tid; u < XT_T * NQ; u += 256) {
    const int tl = u / NQ, q = u % NQ;
    const int64_t t = t0 + tl, g0 = k0 / M + 4 * q;
    const u32x4 pairs = *reinterpret_cast<const u32x4*>(hv + t * 2 * G + 2 * g0);
    const uint32_t nibs = *reinterpret_cast<const uint16_t*>(hm + t * (G / 2) + g0 / 2);
    const u32x4 cs = *reinterpret_cast<const u32x4*>(hc + ((t / V) * G + g0) * 4);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const uint32_t nib = (nibs >> (4 * gi)) & 0xFu;
      const int row = (4 * q + gi) * M;
      const int c0 = (int)((cs[gi] >> (8 * (nib & 3u))) & (uint32_t)(M - 1));
      const int c1 = (int)((cs[gi] >> (8 * (nib >> 2))) & (uint32_t)(M - 1));
      const int r0 = row + c0, r1 = row + c1;
      tile[r0][(((tl >> 3) ^ (r0 >> 4)) & 7) * 8 + (tl & 7)] = (uint16_t)(pairs[gi] & 0xFFFFu);
      tile[r1][(((tl >> 3) ^ (r1 >> 4)) & 7) * 8 + (tl & 7)] = (uint16_t)(pairs[gi] >> 16);
    }
  }
  __syncthreads();
  for (int i = tid; i < XT_F * 8; i += 256) {
    const int r = i >> 3, piece = i & 7;
    *reinterpret_cast<u32x4*>(Ht + (k0 + r) * ldh + t0 + 8 * piece) =
        *reinterpret_cast<const u32x4*>(&tile[r][8 * ((piece ^ (r >> 4)) & 7)]);
  }
}

// Conditions of the vector kernel: whole tiles, a tile's tokens in one V-block, 16-byte rows of
// values and column choices, 2-byte nibble pieces.
static bool expand_vec_ok(const void* hv, const uint8_t* hm, const uint8_t* hc, int64_t Tn, int64_t F, int V, int M,
                          const void* Ht, int64_t ldh) {
  return !env_is_one("NMSPARSE_EXPAND_SCATTER") && Tn % XT_T == 0 && F % XT_F == 0 && V % XT_T == 0 &&
         ldh % 8 == 0 && (uintptr_t)hv % 16 == 0 && (uintptr_t)hm % 2 == 0 && (uintptr_t)hc % 16 == 0 &&
         (uintptr_t)Ht % 16 == 0 && (M == 4 || M == 8 || M == 16);
}

int64_t venom_tn_work_bytes(int esz, int64_t Tn, int64_t F) { return esz == 2 ? F * Tn * 2 : 0; }

hipError_t launch_sddmm_venom(int dt, const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn,
                              int64_t F, int64_t Nc, int V, int M, const void* hv, const uint8_t* hm,
                              const uint8_t* hc, int relu, float* dz, void* dYt, int64_t lddyt, hipStream_t s) {
  if (dt == DT_BF16 && !force_generic() && sddmm_venom_fast_ok(dY, lddy, Wd, ldw, Tn, F, Nc, V, M, hv, dz, dYt, lddyt))
    return launch_sddmm_venom_dma(dY, lddy, Wd, ldw, Tn, F, Nc, V, M, hv, hm, hc, relu, dz, dYt, lddyt, s);
  const int64_t G = F / M;
  const unsigned blocks = (unsigned)((Tn * G + 255) / 256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(sddmm_venom_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)dY, lddy,
                       (const uint16_t*)Wd, ldw, Tn, F, Nc, V, M, (const uint16_t*)hv, hm, hc, relu, dz);
  else
    hipLaunchKernelGGL(sddmm_venom_generic_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, (const uint32_t*)dY, lddy,
                       (const uint32_t*)Wd, ldw, Tn, F, Nc, V, M, (const uint32_t*)hv, hm, hc, relu, dz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dYt) return e;
  return launch_nm_transpose(dt, dY, lddy, Tn, Nc, dYt, lddyt, s);
}

hipError_t launch_spmm_venom_tn(int dt, const void* hv, const uint8_t* hm, const uint8_t* hc, int64_t Tn, int64_t F,
                                int V, int M, const void* dYt, int64_t lddyt, int64_t Nc, float* dW, int64_t lddw,
                                void* work, int64_t work_bytes, hipStream_t s) {
  const int64_t need = venom_tn_work_bytes(dt == DT_BF16 ? 2 : 4, Tn, F);
  if (dt == DT_BF16 && !force_generic() && need > 0 && work && work_bytes >= need && (uintptr_t)work % 16 == 0 &&
      dense_nt_fast_ok(work, Tn, dYt, lddyt, dW, lddw, Tn)) {
    const dim3 grid((unsigned)((Tn + XT_T - 1) / XT_T), (unsigned)((F + XT_F - 1) / XT_F));
    if (expand_vec_ok(hv, hm, hc, Tn, F, V, M, work, Tn)) {
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const uint16_t*)hv, hm, hc, F, V, (uint16_t*)work, Tn);
      };
      if (M == 4) go(venom_expand_t_vec_kernel<4>);
      else if (M == 8) go(venom_expand_t_vec_kernel<8>);
      else go(venom_expand_t_vec_kernel<16>);
    } else {
      hipLaunchKernelGGL(venom_expand_t_kernel, grid, dim3(256), 0, s, (const uint16_t*)hv, hm, hc, Tn, F, V, M,
                         (uint16_t*)work, Tn);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dense_nt(work, Tn, dYt, lddyt, F, Nc, Tn, dW, lddw, s);
  }
  const unsigned blocks = (unsigned)((F * Nc + 255) / 256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(spmm_venom_tn_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)hv, hm,
                       hc, Tn, F, V, M, (const uint16_t*)dYt, lddyt, Nc, dW, lddw);
  else
    hipLaunchKernelGGL(spmm_venom_tn_generic_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, (const uint32_t*)hv, hm,
                       hc, Tn, F, V, M, (const uint32_t*)dYt, lddyt, Nc, dW, lddw);
  return hipGetLastError();
}

}  // namespace nms
