// Weight gradient of a 2:4 layer sampled at the weight's survivors (gfx950).
//
// "Success story: ESPLAG" (Research Topic) needed kernels beyond the SpMM for
// the complete sparse training step.  For Y = W_s X the weight gradient is
// dY X^T, and only the entries W_s keeps are needed:
//   out[r][2g+s] = sum_t D[r][t] * X[4g + p_s(r, g)][t],   D = dY.
// Which two of each four outputs survive varies per row, so the matrix
// instruction cannot skip work: the kernel is a dense bf16 "NT" GEMM (both
// operands contiguous along the reduction index t, so no transposes), with the
// selection done in the epilogue.
//
// v_mfma_f32_16x16x32_bf16 on gfx950: lane l holds row l%16 of A and column
// l%16 of B, k = 8*(l/16)..+7; the result holds column l%16, rows
// 4*(l/16)..+3.  Fragment j of each 64-column group maps lane c to output
// column 4c + j, so every lane ends up holding all four columns of one 2:4
// group of the weight: the selection is lane-local (two of the lane's four
// accumulators, chosen by the group's nibble), and the 16 lanes of a row write
// 16 consecutive float2 pairs -- 128 contiguous bytes.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {

// ---------------------------------------------------------------------------
// generic path: any dtype / alignment.  64 x 64 dense tile over (r, c).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void sddmm_generic_kernel(const T* __restrict__ D, int64_t ldd, const T* __restrict__ X,
                                                            int64_t ldx, int64_t R, int64_t Kc, int64_t Tn,
                                                            const uint8_t* __restrict__ meta, float* __restrict__ out) {
  constexpr int TM = 64, TN = 64, KC = 32;
  __shared__ float Ds[KC][TM + 4];
  __shared__ float Xs[KC][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < Tn; t0 += KC) {
    for (int i = tid; i < KC * TM; i += 256) {
      const int r = i / KC, kk = i % KC;
      const int64_t row = m0 + r, t = t0 + kk;
      Ds[kk][r] = (row < R && t < Tn) ? Elem<T>::to_f32(D[row * ldd + t]) : 0.f;
      const int64_t col = n0 + r;
      Xs[kk][r] = (col < Kc && t < Tn) ? Elem<T>::to_f32(X[col * ldx + t]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Ds[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Xs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  // lane (ty, tx) holds columns n0 + 4tx .. +3: one whole 2:4 group
  const int64_t gq = n0 / 4 + tx;
  if (gq >= Kc / 4) return;
  const int64_t mrow = (Kc + 7) / 8;
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= R) continue;
    const uint32_t nib = (meta[row * mrow + gq / 2] >> (4 * (gq & 1))) & 0xF;
    out[row * (Kc / 2) + 2 * gq] = acc[i][nib & 3];
    out[row * (Kc / 2) + 2 * gq + 1] = acc[i][(nib >> 2) & 3];
  }
}

// ---------------------------------------------------------------------------
// fast path: bf16 v_mfma_f32_16x16x32_bf16
// ---------------------------------------------------------------------------
constexpr int DK = 64;        // t per k-step
constexpr int D_PITCH = 72;   // u16 per LDS row (64 + 8 pad)

__device__ inline int sd_lds_row(int n) { return (n & ~63) | ((n & 3) << 4) | ((n & 63) >> 2); }

template <int BM, int BN, int WM, int WN>
struct SddmmCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_CH = BM * 8 / NT;     // 16-byte chunks of D per lane per k-step
  static constexpr int B_CH = BN * 8 / NT;     // 16-byte chunks of X per lane per k-step
  static constexpr int LDS_A = BM * D_PITCH * 2;
  static constexpr int LDS_B = BN * D_PITCH * 2;
  static constexpr int STAGE = LDS_A + LDS_B;
  static_assert(WN % 64 == 0, "whole 64-column groups per wave");
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "chunking");
  static_assert(NT == 256, "kernels are compiled for 256-lane workgroups");
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void sddmm_mfma_kernel(
    const uint16_t* __restrict__ D, int64_t ldd, const uint16_t* __restrict__ X, int64_t ldx, int64_t R, int64_t Kc,
    int64_t Tn, const uint8_t* __restrict__ meta, float* __restrict__ out) {
  using Cfg = SddmmCfg<BM, BN, WM, WN>;
  constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Kc + BN - 1) / BN);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  constexpr int GM = 8;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int KT = (int)((Tn + DK - 1) / DK);

  u32x4 ra[Cfg::A_CH], rb[Cfg::B_CH];
  auto load_global = [&](int kt) {
    const int64_t t0 = (int64_t)kt * DK;
#pragma unroll
    for (int i = 0; i < Cfg::A_CH; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3, part = c & 7;
      const int64_t row = m0 + r, t = t0 + part * 8;
      ra[i] = (row < R && t < Tn) ? *reinterpret_cast<const u32x4*>(D + row * ldd + t) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_CH; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 3, part = c & 7;
      const int64_t col = n0 + r, t = t0 + part * 8;
      rb[i] = (col < Kc && t < Tn) ? *reinterpret_cast<const u32x4*>(X + col * ldx + t) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int buf) {
    unsigned char* st = smem + buf * Cfg::STAGE;
    uint16_t* As = reinterpret_cast<uint16_t*>(st);
    uint16_t* Bs = reinterpret_cast<uint16_t*>(st + Cfg::LDS_A);
#pragma unroll
    for (int i = 0; i < Cfg::A_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4*>(As + (c >> 3) * D_PITCH + (c & 7) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_CH; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4*>(Bs + sd_lds_row(c >> 3) * D_PITCH + (c & 7) * 8) = rb[i];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lr16 = lane & 15, lg = lane >> 4;

  auto compute = [&](int buf) {
    const unsigned char* st = smem + buf * Cfg::STAGE;
    const uint16_t* As = reinterpret_cast<const uint16_t*>(st);
    const uint16_t* Bs = reinterpret_cast<const uint16_t*>(st + Cfg::LDS_A);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 a[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * WM + i * 16 + lr16) * D_PITCH + kh * 32 + lg * 8);
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int lrow = wn * WN + (f >> 2) * 64 + (f & 3) * 16 + lr16;
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bs + lrow * D_PITCH + kh * 32 + lg * 8);
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][f], 0, 0, 0);
      }
    }
  };

  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    compute(cur);
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds the 4 columns of group gq for rows 16i + 4lg + e
  const int64_t mrow = (Kc + 7) / 8;
  const int64_t G = Kc / 4;
#pragma unroll
  for (int grp4 = 0; grp4 < FN / 4; ++grp4) {
    const int64_t gq = (n0 + wn * WN + grp4 * 64) / 4 + lr16;
    if (gq >= G) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * WM + i * 16 + lg * 4 + e;
        if (row >= R) continue;
        const uint32_t nib = (meta[row * mrow + gq / 2] >> (4 * (gq & 1))) & 0xF;
        float v[4] = {acc[i][grp4 * 4 + 0][e], acc[i][grp4 * 4 + 1][e], acc[i][grp4 * 4 + 2][e],
                      acc[i][grp4 * 4 + 3][e]};
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        f32x2 o = {v[nib & 3], v[(nib >> 2) & 3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x2*>(out + row * (Kc / 2) + 2 * gq));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// pipelined path: direct-to-LDS loads, v_mfma_f32_16x16x32_bf16.
//
// A wave owns WM rows x 128 output columns as 16 x 16 fragments; fragment j
// (of 8) maps lane c (= l % 16) to output column 64 (j / 4) + 4 c + j % 4, so
// every lane holds all four columns of its 2:4 groups and selects two of them
// by the group's nibble.  Tiles are staged per 64 t (128-byte rows, whole
// cache lines) in two buffers, loaded with direct-to-LDS dwordx4 loads; X rows
// are placed so that each fragment's 16 rows are consecutive in LDS, and the
// 16-byte chunks of LDS row r are XOR-swizzled by (r >> 1) & 7, which keeps the
// ds_read_b128 operand reads of 16 consecutive rows free of bank conflicts.
// ---------------------------------------------------------------------------
constexpr int TK = 64;   // t per stage

__device__ __forceinline__ int sd_swz(int r) { return (r >> 1) & 7; }

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
struct SdCfg {
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int A_BYTES = BM * TK * 2, B_BYTES = BN * TK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / NW, B_INSTR = B_BYTES / 1024 / NW;
  static constexpr int LOADS = A_INSTR + B_INSTR;
  static_assert(WN == 128, "a wave owns 128 output columns (32 whole 2:4 groups)");
  static_assert(WM % 32 == 0 && A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "tiling");
  static_assert(STAGES == 2 && STAGE * STAGES <= 160 * 1024, "two LDS buffers");
};

// WRITE_DT: the kernel also writes Dt[t][r] = D[r][t].  Every 64-t stage of a BM-row panel of D
// passes through the LDS of all the panel's column tiles; the one with column tile
// tn == kt % (number of column tiles) transposes stage kt from LDS -- waves 0 .. BM/64 - 1, one
// 8 x 8 block per lane (eight 16-byte LDS reads, v_perm, eight 16-byte stores; the 8 lanes of a t
// row write 128 contiguous bytes) -- so each stage is written once and the work is spread evenly.
//
// MODE: SD_NM -- out[r][2g+s] = (D X^T)[r][4g + p_s(r, g)], p_s from the 2:4 nibbles `meta` (the
//   weight gradient of a 2:4 layer);
// SD_VNM -- the columns of X are the rows gathered through a V:N:M column selection: gathered
//   column 4g + j is row g*M + colsel[r/V][g][j] of X (the tile's BM rows lie in one V-block), and
//   out[r][2g+s] = (D X_gathered^T)[r][4g + j_s(r, g)] with j_s from the V:N:M nibbles `meta`,
//   set to 0 where hval[r][2g+s] (bf16) is not > 0 when relu (the gradient of ReLU'd V:N:M
//   activations);
// SD_DENSE -- out[r][c] = (D X^T)[r][c] for every column, row stride ldo (a plain NT GEMM).
enum { SD_NM = 0, SD_VNM = 1, SD_DENSE = 2 };

// Epilogue of the pipelined SDDMM kernels: a wave's FM x 8 accumulator fragments of 16 x 16 cover
// rows r0w .. r0w + 16 FM - 1 and 128 output columns from c0w; lane l holds rows 16 i + 4 (l / 16) + e
// (e < 4) and, in fragment j, column c0w + 64 (j / 4) + 4 (l % 16) + j % 4, so lanes hold every column
// of 2:4 groups c0w/4 + 16 q + l % 16 (q < 2).  SD_DENSE stores all four (16 bytes per row), the other
// modes the two the nibble keeps (8 bytes per row).
template <int FM, int MODE>
__device__ __forceinline__ void sd_epilogue16x(const f32x4 (&acc)[FM][8], int64_t r0w, int64_t c0w, int l16, int aq,
                                               int64_t R, int64_t Kc, const uint8_t* __restrict__ meta,
                                               float* __restrict__ out, const uint16_t* __restrict__ hval, int relu,
                                               int64_t ldo) {
  const int64_t G = Kc / 4, mrow = (Kc + 7) / 8;
  const int64_t mrow_v = MODE == SD_VNM ? (G + 1) / 2 : mrow;   // V:N:M nibbles: one per gathered group
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t gq = c0w / 4 + 16 * q + l16;
    if constexpr (MODE == SD_DENSE) {
      const int64_t c0 = 4 * gq;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = r0w + 16 * i + 4 * aq + e;
          if (row < R && c0 < Kc) {
            float* dst = out + row * ldo + c0;
            const float v[4] = {acc[i][4 * q][e], acc[i][4 * q + 1][e], acc[i][4 * q + 2][e], acc[i][4 * q + 3][e]};
            if (c0 + 4 <= Kc) {
              __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(dst));
            } else {
              for (int u = 0; u < 4 && c0 + u < Kc; ++u) dst[u] = v[u];
            }
          }
        }
    } else {
      if (gq < G) {
        uint32_t mb[FM][4];   // the metadata byte of every output row of the lane, loaded up front
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int64_t row = r0w + 16 * i + 4 * aq + e;
            row = row < R ? row : R - 1;
            mb[i][e] = meta[row * mrow_v + gq / 2];
          }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t row = r0w + 16 * i + 4 * aq + e;
            if (row < R) {
              const uint32_t nib = (mb[i][e] >> (4 * (gq & 1))) & 0xF;
              const float v0 = acc[i][4 * q][e], v1 = acc[i][4 * q + 1][e], v2 = acc[i][4 * q + 2][e],
                          v3 = acc[i][4 * q + 3][e];
              const uint32_t p0 = nib & 3, p1 = (nib >> 2) & 3;
              typedef float f32x2 __attribute__((ext_vector_type(2)));
              f32x2 o;
              o[0] = p0 == 0 ? v0 : p0 == 1 ? v1 : p0 == 2 ? v2 : v3;
              o[1] = p1 == 0 ? v0 : p1 == 1 ? v1 : p1 == 2 ? v2 : v3;
              if constexpr (MODE == SD_VNM) {
                if (relu) {
                  // ReLU's derivative at the kept activations: 1 where the bf16 value is > 0
                  const uint32_t hp = *reinterpret_cast<const uint32_t*>(hval + row * (2 * G) + 2 * gq);
                  o[0] = Elem<uint16_t>::positive((uint16_t)(hp & 0xFFFF)) ? o[0] : 0.f;
                  o[1] = Elem<uint16_t>::positive((uint16_t)(hp >> 16)) ? o[1] : 0.f;
                }
              }
              __builtin_nontemporal_store(o, reinterpret_cast<f32x2*>(out + row * (Kc / 2) + 2 * gq));
            }
          }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool WRITE_DT, int MODE = SD_NM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void sddmm_dma_kernel(
    const uint16_t* __restrict__ D, int64_t ldd, const uint16_t* __restrict__ X, int64_t ldx, int64_t R, int64_t Kc,
    int64_t Tn, const uint8_t* __restrict__ meta, float* __restrict__ out, uint16_t* __restrict__ Dt, int64_t lddt,
    const uint8_t* __restrict__ colsel, int V, int M, const uint16_t* __restrict__ hval, int relu, int64_t ldo) {
  using Cfg = SdCfg<BM, BN, WAVES_M, WAVES_N, STAGES>;
  static_assert(!WRITE_DT || BM % 64 == 0, "transposing waves cover 64 rows each");
  static_assert(!WRITE_DT || BM / 64 <= WAVES_M * WAVES_N, "enough waves to transpose a stage");
  constexpr int FM = Cfg::WM / 16, FN = 8;   // 16 x 16 fragments of the wave's WM x 128
  extern __shared__ __align__(1024) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Kc + BN - 1) / BN);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  constexpr int GM = 4;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int KT = (int)(Tn / TK);
  const uint32_t smem_base = lds_addr(smem);

  // DMA sources: instruction q covers LDS bytes q*1024.. = 8 rows of 128 bytes;
  // lane -> LDS row 8q + lane/8, chunk position lane%8 (holding chunk pos ^ swz)
  const uint16_t* a_src[Cfg::A_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::A_INSTR; ++t) {
    const int r = 8 * (wave * Cfg::A_INSTR + t) + (lane >> 3);
    const int c = (lane & 7) ^ sd_swz(r);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    a_src[t] = D + row * ldd + 8 * c;
  }
  const uint16_t* b_src[Cfg::B_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::B_INSTR; ++t) {
    const int r = 8 * (wave * Cfg::B_INSTR + t) + (lane >> 3);      // LDS row
    const int c = (lane & 7) ^ sd_swz(r);
    const int n = (r & ~63) | ((r & 15) << 2) | ((r >> 4) & 3);   // tile column of LDS row r
    int64_t col = n0 + n;
    col = col < Kc ? col : Kc - 1;
    if constexpr (MODE == SD_VNM) {
      // gathered column -> row of X through the tile's V-block's column selection
      const int64_t g = col >> 2, G = Kc >> 2;
      col = g * M + (colsel[((m0 / V) * G + g) * 4 + (col & 3)] & (M - 1));
    }
    b_src[t] = X + col * ldx + 8 * c;
  }
  auto issue = [&](int kt) {
    const uint32_t st = smem_base + (kt % STAGES) * Cfg::STAGE;
    const int64_t t0 = (int64_t)kt * TK;
#pragma unroll
    for (int t = 0; t < Cfg::A_INSTR; ++t) dma16(a_src[t] + t0, uniform(st + (wave * Cfg::A_INSTR + t) * 1024));
#pragma unroll
    for (int t = 0; t < Cfg::B_INSTR; ++t)
      dma16(b_src[t] + t0, uniform(st + Cfg::A_BYTES + (wave * Cfg::B_INSTR + t) * 1024));
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  const int l16 = lane & 15, aq = lane >> 4;
  // fragments' rows start at multiples of 16: one per-lane base and swizzle per operand
  const int a_base = (wm * Cfg::WM + l16) * (TK * 2), b_base = Cfg::A_BYTES + (wn * 128 + l16) * (TK * 2);
  const int swz = sd_swz(l16);
  // A stage is two 32-t sub-steps of 8 x FM v_mfma_f32_16x16x32_bf16 (lane l: row (column) l % 16 of
  // a fragment, t = 32 kk + 8 (l / 16) .. +7).  One register set of operands (two waves per SIMD hide
  // each other's LDS latency; a second set would not fit beside the transposes' registers).  The
  // accumulators are tied through the instruction in assembly (as builtins, the compiler moves the
  // small accumulators between registers every stage).
  auto read_ops = [&](const unsigned char* st, int kk, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
    const int co = (((4 * kk + aq) ^ swz) << 4);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj)
      b[jj] = *reinterpret_cast<const bf16x8*>(st + b_base + co + jj * 16 * (TK * 2));
#pragma unroll
    for (int ii = 0; ii < FM; ++ii)
      a[ii] = *reinterpret_cast<const bf16x8*>(st + a_base + co + ii * 16 * (TK * 2));
  };
  auto mma = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN]) {
#pragma unroll
    for (int jj = 0; jj < FN; ++jj)
#pragma unroll
      for (int ii = 0; ii < FM; ++ii)
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[ii][jj]) : "v"(a[ii]), "v"(b[jj]));
  };
  auto compute = [&](int kt) {
    const unsigned char* st = smem + (kt % STAGES) * Cfg::STAGE;
    bf16x8 a0[FM], b0[FN];
    read_ops(st, 0, a0, b0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    read_ops(st, 1, a0, b0);
    mma(a0, b0);
  };

  // Dt: stage kt of this row panel is written by the workgroup whose column tile is kt % ntn
  constexpr int kDtStores = 8;   // 16-byte stores per lane of a transposing wave and stage
  auto transpose_stage = [&](int kt) {
    // waves 0 .. BM/64 - 1: BM/8 row blocks x 8 t blocks of 8 x 8; the 8 lanes of a row block
    // read the 8 chunks of each of its rows (the whole 128-byte LDS row: no bank conflicts)
    const int tb = lane & 7, rb = 8 * wave + (lane >> 3);
    const unsigned char* st = smem + (kt % STAGES) * Cfg::STAGE;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * rb + i;
      v[i] = *reinterpret_cast<const u32x4*>(st + r * (TK * 2) + ((tb ^ sd_swz(r)) << 4));
    }
    const int64_t col = m0 + 8 * rb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = __builtin_amdgcn_perm(v[2 * j + 1][e >> 1], v[2 * j][e >> 1], sel);
      uint16_t* dst = Dt + ((int64_t)kt * TK + 8 * tb + e) * lddt + col;
      if (col + 8 <= R) {
        // non-temporal: the 268 MB of a training step's dY^T would otherwise push the SDDMM's
        // operands out of L2 (about 2% slower with ordinary stores)
        __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(dst));
      } else {
        // rows past R (a partial last panel) are never written
        for (int q = 0; q < 8; ++q)
          if (col + q < R) dst[q] = (uint16_t)(d[q >> 1] >> (16 * (q & 1)));
      }
    }
  };

  // two buffers: the loads of stage kt+1 are in flight while stage kt runs on the matrix cores
  if (KT > 0) issue(0);
  // A transposing wave of a whole row panel issues exactly kDtStores stores (one 16-byte store
  // per e, every lane in range), younger than its loads of the next stage, so waiting until only
  // kDtStores operations are outstanding covers those loads.  In a partial last panel a wave may
  // issue fewer stores (none at all when every one of its rows lies past R), so there every wait
  // is for all outstanding operations.
  const bool whole_panel = m0 + BM <= R;
  bool wrote = false;   // this wave stored a transposed stage of a whole panel during the previous step
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of stage kt have landed (after a transposing step the stores of that step,
    // which are younger than those loads, may still be in flight)
    if (WRITE_DT && wrote) wait_vmcnt<kDtStores>(); else wait_vmcnt<0>();
    lds_barrier();     // ... every wave's; and every wave is done reading stage kt-1 (the other buffer)
    if (kt + 1 < KT) issue(kt + 1);
    compute(kt);
    wrote = false;
    if (WRITE_DT && kt % ntn == tn && wave < BM / 64) {
      transpose_stage(kt);
      wrote = whole_panel;
    }
  }
  if (WRITE_DT) wait_vmcnt<0>();

  // the last instructions' results before any other instruction reads them (the compiler does not
  // see the instructions inside the assembly statements)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  sd_epilogue16x<FM, MODE>(acc, m0 + wm * Cfg::WM, n0 + wn * 128, l16, aq, R, Kc, meta, out, hval, relu, ldo);
}

// ---------------------------------------------------------------------------
// Four-wave path: 128 x 128 per wave on a 256 x 256 tile, the memory instructions issued between
// the matrix instructions.
//
// Two LDS buffers of one 64-t stage (2 x 64 KB), filled by direct-to-LDS loads of whole 128-byte
// rows (the swizzle of the kernel above, sd_swz; X rows placed so that every lane's fragments
// hold the four columns of its 2:4 groups).  A stage is two 32-t sub-steps of 64
// v_mfma_f32_16x16x32_bf16 per wave (8 x 8 fragments of 16 x 16); after every fourth matrix
// instruction the wave reads one operand of the next sub-step from LDS, so no sub-step waits for
// its operands.  The barrier sits between the two sub-steps: by then every wave has read all of
// the stage, so the second sub-step reads the next stage's first operands, and the buffer just
// left takes the loads of the stage after next: half of them during that sub-step, the other half
// during the next stage's first, one after every fourth matrix instruction of the first 32 (issued
// faster, they queue in the vector-memory address unit and hold the wave at the issue of the
// next).  One wave per SIMD: a wave's 256 fp32 accumulators sit in the accumulation registers.
// Under the chip's power limit the 16 x 16 x 32 instruction sustains ~10% more flops than the
// 32 x 32 x 16 one (1784 against 1617 TFLOP/s in loops of nothing else on changing operands).
// ---------------------------------------------------------------------------
constexpr int W4_A = 256 * TK * 2, W4_STAGE = 2 * W4_A;   // D and X parts of a stage: 32 KB each

template <bool WRITE_DT, int MODE>
__global__ __launch_bounds__(256) void sddmm_w4_kernel(const uint16_t* __restrict__ D, int64_t ldd,
                                                        const uint16_t* __restrict__ X, int64_t ldx, int64_t R,
                                                        int64_t Kc, int64_t Tn, const uint8_t* __restrict__ meta,
                                                        float* __restrict__ out, uint16_t* __restrict__ Dt,
                                                        int64_t lddt, int64_t ldo) {
  static_assert(MODE == SD_NM || MODE == SD_DENSE, "the gathered (V:N:M) mode keeps the eight-wave kernel");
  constexpr int FM = 8, FN = 8;   // 16 x 16 fragments of the wave's 128 x 128
  extern __shared__ __align__(1024) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int ntm = (int)((R + 255) / 256), ntn = (int)((Kc + 255) / 256);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  constexpr int GM = 4;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * 256, n0 = (int64_t)tn * 256;
  const int KT = (int)(Tn / TK);

  // load t of a wave: LDS rows 8 (8 wave + t) .. +7 of the D part (t < 8) or of the X part;
  // lane -> row 8 (8 wave + t) + lane / 8, LDS chunk lane % 8 holding source chunk (lane % 8) ^ swz.
  // Sources are 32-bit byte offsets from the stage's wave-uniform base (the dispatch checks that
  // both operands are smaller than 4 GiB).
  uint32_t off[16];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int r = 8 * (8 * wave + t) + (lane >> 3);
    const int c = (lane & 7) ^ sd_swz(r);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    off[t] = (uint32_t)(2 * (row * ldd + 8 * c));
    const int n = (r & ~63) | ((r & 15) << 2) | ((r >> 4) & 3);   // tile column of LDS row r
    int64_t col = n0 + n;
    col = col < Kc ? col : Kc - 1;
    off[8 + t] = (uint32_t)(2 * (col * ldx + 8 * c));
  }
  const uint32_t lds_wave = lds_addr(smem) + (8 * wave) * 1024;
  // load t (< 16) of stage kl into LDS buffer buf
  auto dma = [&](int t, int kl, int buf) {
    const uint16_t* base = (t < 8 ? D : X) + (int64_t)kl * TK;
    dma16s(off[t], base, uniform(lds_wave + buf * W4_STAGE + (t < 8 ? 0 : W4_A) + (t & 7) * 1024));
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  const int l16 = lane & 15, aq = lane >> 4;
  // Fragment i's rows start at a multiple of 16, so every fragment's row l16 has the swizzle
  // sd_swz(l16): one per-lane base per operand, fragments and buffers as constant offsets.
  const int a_base = (wm * 128 + l16) * (TK * 2), b_base = W4_A + (wn * 128 + l16) * (TK * 2);
  const int swz = sd_swz(l16);
  // operand q of sub-step kk (32 t; q < 8: A fragment q, else B fragment q - 8): lane l holds row
  // (column) l % 16 of the fragment, t = 32 kk + 8 (l / 16) .. +7
  auto read_op = [&](int buf, int kk, int q, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
    const int co = buf * W4_STAGE + (((4 * kk + aq) ^ swz) << 4);
    if (q < 8)
      a[q] = *reinterpret_cast<const bf16x8*>(smem + a_base + co + q * 16 * (TK * 2));
    else
      b[q - 8] = *reinterpret_cast<const bf16x8*>(smem + b_base + co + (q - 8) * 16 * (TK * 2));
  };
  // One 32-t sub-step: 64 matrix instructions on (a, b), B fragment j outer; after every fourth,
  // one LDS read of the next operands (operand m/4 of sub-step kk_next of buffer rbuf, into
  // an / bn; the A fragments first, none when kk_next < 0), and after every fourth from the
  // second on (the first 32 only) other(0 .. 7): loads of a stage in flight.  Scheduling barriers
  // keep this order, so that each memory instruction issues while a matrix instruction runs.
  auto substep = [&](const bf16x8 (&a)[FM], const bf16x8 (&b)[FN], int rbuf, int kk_next, bf16x8 (&an)[FM],
                     bf16x8 (&bn)[FN], auto other) {
#pragma unroll
    for (int m = 0; m < 64; ++m) {
      const int j = m >> 3, i = m & 7;
      // the accumulator tied in and out of the instruction in the accumulation registers (as a
      // builtin, the compiler moves the 64 small accumulators between registers every iteration)
      asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(a[i]), "v"(b[j]));
      __builtin_amdgcn_sched_barrier(0);
      if ((m & 3) == 0 && kk_next >= 0) read_op(rbuf, kk_next, m >> 2, an, bn);
      if ((m & 3) == 2 && m < 32) other(m >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Dt: stage kt of this row panel is written by the workgroup whose column tile is kt % ntn; all
  // four waves, one 8 x 8 block per lane (as in the direct-to-LDS kernel)
  auto transpose_stage = [&](int kt) {
    const int tb = lane & 7, rb = 8 * wave + (lane >> 3);
    const unsigned char* st = smem + (kt & 1) * W4_STAGE;
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * rb + i;
      v[i] = *reinterpret_cast<const u32x4*>(st + r * (TK * 2) + ((tb ^ sd_swz(r)) << 4));
    }
    const int64_t col = m0 + 8 * rb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = __builtin_amdgcn_perm(v[2 * j + 1][e >> 1], v[2 * j][e >> 1], sel);
      uint16_t* dst = Dt + ((int64_t)kt * TK + 8 * tb + e) * lddt + col;
      if (col + 8 <= R) {
        __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(dst));
      } else {
        for (int q = 0; q < 8; ++q)
          if (col + q < R) dst[q] = (uint16_t)(d[q >> 1] >> (16 * (q & 1)));
      }
    }
  };

  // Stage kt (a0 / b0: its sub-step-0 operands, read during the previous stage).  The wait before
  // the barrier is for stage kt+1's loads (issued during the previous stage's last sub-step);
  // a transposing wave's Dt stores of this stage are younger than them and may stay in flight
  // (a whole panel's wave issues exactly kDtStores; in a partial last panel every wait is for all).
  constexpr int kDtStores = 8;
  const bool whole_panel = m0 + 256 <= R;
  auto stage = [&](int kt, bf16x8 (&a0)[FM], bf16x8 (&b0)[FN]) {
    const int buf = kt & 1;
    bf16x8 a1[FM], b1[FN];
    const int kn = kt + 1 < KT ? kt + 1 : KT - 1;   // past the end: a repeat that is never read
    substep(a0, b0, buf, 1, a1, b1, [&](int t) { dma(8 + t, kn, buf ^ 1); });
    bool wrote = false;
    if constexpr (WRITE_DT) {
      if (kt % ntn == tn) {
        transpose_stage(kt);
        wrote = whole_panel;
      }
    }
    if (wrote) wait_vmcnt<kDtStores>(); else wait_vmcnt<0>();
    lds_barrier();   // stage kt+1 is in LDS for every wave; every wave has read all it needs of stage kt
    const int kl = kt + 2 < KT ? kt + 2 : KT - 1;   // past the end: a repeat that is never read
    substep(a1, b1, buf ^ 1, 0, a0, b0, [&](int t) { dma(t, kl, buf); });
  };

  // KT is even and at least 2 (the dispatch checks Tn % 128 == 0)
#pragma unroll
  for (int t = 0; t < 16; ++t) dma(t, 0, 0);
#pragma unroll
  for (int t = 0; t < 8; ++t) dma(t, 1, 1);
  wait_vmcnt<8>();   // stage 0
  lds_barrier();
  bf16x8 a0[FM], b0[FN];
#pragma unroll
  for (int q = 0; q < 16; ++q) read_op(0, 0, q, a0, b0);
  for (int kt = 0; kt < KT; kt += 2) {
    stage(kt, a0, b0);
    stage(kt + 1, a0, b0);
  }
  wait_vmcnt<0>();   // drain: no load may land in LDS after the workgroup ends

  // the last matrix instructions' results before any other instruction reads them (the compiler does
  // not see the instructions inside the assembly statements)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  sd_epilogue16x<8, MODE>(acc, m0 + wm * 128, n0 + wn * 128, l16, aq, R, Kc, meta, out, nullptr, 0, ldo);
}

template <bool WRITE_DT, int MODE>
static hipError_t run_sddmm_w4(const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                                int64_t Tn, const uint8_t* meta, float* out, void* Dt, int64_t lddt, int64_t ldo,
                                hipStream_t s) {
  const size_t lds = 2 * (size_t)W4_STAGE;
  auto kern = sddmm_w4_kernel<WRITE_DT, MODE>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + 255) / 256) * ((Kc + 255) / 256);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(256), lds, s, (const uint16_t*)D, ldd, (const uint16_t*)X,
                     ldx, R, Kc, Tn, meta, out, (uint16_t*)Dt, lddt, ldo);
  return hipGetLastError();
}

// The four-wave kernel takes pairs of 64-t stages and addresses each operand with 32-bit
// byte offsets from its base.
static bool sd_w4_ok(int64_t R, int64_t ldd, int64_t Kc, int64_t ldx, int64_t Tn) {
  if (env_is_one("NMSPARSE_SDDMM_DMA")) return false;
  return Tn % (2 * TK) == 0 && R * ldd * 2 < (int64_t(1) << 32) && Kc * ldx * 2 < (int64_t(1) << 32);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool WRITE_DT, int MODE = SD_NM>
static hipError_t run_sddmm_dma(const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                                int64_t Tn, const uint8_t* meta, float* out, void* Dt, int64_t lddt, hipStream_t s,
                                const uint8_t* colsel = nullptr, int V = 1, int M = 4, const void* hval = nullptr,
                                int relu = 0, int64_t ldo = 0) {
  using Cfg = SdCfg<BM, BN, WAVES_M, WAVES_N, STAGES>;
  const size_t lds = (size_t)Cfg::STAGE * STAGES;
  auto kern = sddmm_dma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, WRITE_DT, MODE>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Kc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), lds, s, (const uint16_t*)D, ldd, (const uint16_t*)X,
                     ldx, R, Kc, Tn, meta, out, (uint16_t*)Dt, lddt, colsel, V, M, (const uint16_t*)hval, relu, ldo);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t run_sddmm_mfma(const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                                 int64_t Tn, const uint8_t* meta, float* out, hipStream_t s) {
  using Cfg = SddmmCfg<BM, BN, WM, WN>;
  const size_t lds = 2 * (size_t)Cfg::STAGE;
  auto kern = sddmm_mfma_kernel<BM, BN, WM, WN>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Kc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), lds, s, (const uint16_t*)D, ldd, (const uint16_t*)X,
                     ldx, R, Kc, Tn, meta, out);
  return hipGetLastError();
}

hipError_t launch_sddmm_nm(int dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                           int64_t Tn, const uint8_t* meta, float* out, hipStream_t s) {
  const char* e = getenv("NMSPARSE_FORCE_GENERIC");
  const bool force = e && e[0] == '1';
  const char* tier = getenv("NMSPARSE_SPMM_TIER");
  const bool staged = tier && tier[0] == '1';
  if (dt == DT_BF16 && !force && !staged && Tn % TK == 0 && ldd % 8 == 0 && ldx % 8 == 0 && (uintptr_t)D % 16 == 0 &&
      (uintptr_t)X % 16 == 0 && (uintptr_t)out % 8 == 0)
    return sd_w4_ok(R, ldd, Kc, ldx, Tn)
               ? run_sddmm_w4<false, SD_NM>(D, ldd, X, ldx, R, Kc, Tn, meta, out, nullptr, 0, 0, s)
               : run_sddmm_dma<256, 256, 4, 2, 2, false>(D, ldd, X, ldx, R, Kc, Tn, meta, out, nullptr, 0, s);
  if (dt == DT_BF16 && !force && Tn % 8 == 0 && ldd % 8 == 0 && ldx % 8 == 0 && (uintptr_t)D % 16 == 0 &&
      (uintptr_t)X % 16 == 0 && (uintptr_t)out % 8 == 0)
    return run_sddmm_mfma<256, 128, 128, 64>(D, ldd, X, ldx, R, Kc, Tn, meta, out, s);
  dim3 grid((unsigned)((Kc + 63) / 64), (unsigned)((R + 63) / 64));
  if (dt == DT_BF16)
    hipLaunchKernelGGL(sddmm_generic_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)D, ldd,
                       (const uint16_t*)X, ldx, R, Kc, Tn, meta, out);
  else
    hipLaunchKernelGGL(sddmm_generic_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)D, ldd,
                       (const uint32_t*)X, ldx, R, Kc, Tn, meta, out);
  return hipGetLastError();
}

// sddmm_nm that also writes Dt = D^T [Tn][lddt]: one kernel on the pipelined path, otherwise the
// SDDMM followed by the transpose.
hipError_t launch_sddmm_nm_dt(int dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                              int64_t Tn, const uint8_t* meta, float* out, void* Dt, int64_t lddt, hipStream_t s) {
  if (dt == DT_BF16 && !force_generic() && !env_is_one("NMSPARSE_SPMM_TIER") && Tn % TK == 0 && ldd % 8 == 0 &&
      ldx % 8 == 0 && (uintptr_t)D % 16 == 0 && (uintptr_t)X % 16 == 0 && (uintptr_t)out % 8 == 0 &&
      (uintptr_t)Dt % 16 == 0 && lddt % 8 == 0)
    return sd_w4_ok(R, ldd, Kc, ldx, Tn)
               ? run_sddmm_w4<true, SD_NM>(D, ldd, X, ldx, R, Kc, Tn, meta, out, Dt, lddt, 0, s)
               : run_sddmm_dma<256, 256, 4, 2, 2, true>(D, ldd, X, ldx, R, Kc, Tn, meta, out, Dt, lddt, s);
  const hipError_t e = launch_sddmm_nm(dt, D, ldd, X, ldx, R, Kc, Tn, meta, out, s);
  if (e != hipSuccess) return e;
  return launch_nm_transpose(dt, D, ldd, R, Tn, Dt, lddt, s);
}

// V:N:M SDDMM (gradient of V:N:M activations): 128 x 512 tiles (128 tokens inside one V-block,
// 512 gathered columns), eight waves of 64 x 128, two stages of 80 KB.
bool sddmm_venom_fast_ok(const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn, int64_t F, int64_t Nc,
                         int V, int M, const void* hv, const float* dz, const void* dYt, int64_t lddyt) {
  (void)Tn, (void)F, (void)M;
  return Nc % TK == 0 && V % 128 == 0 && lddy % 8 == 0 && ldw % 8 == 0 && (uintptr_t)dY % 16 == 0 &&
         (uintptr_t)Wd % 16 == 0 && (uintptr_t)dz % 8 == 0 && (uintptr_t)hv % 4 == 0 &&
         (!dYt || ((uintptr_t)dYt % 16 == 0 && lddyt % 8 == 0));
}

hipError_t launch_sddmm_venom_dma(const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn, int64_t F,
                                  int64_t Nc, int V, int M, const void* hv, const uint8_t* hm, const uint8_t* hc,
                                  int relu, float* dz, void* dYt, int64_t lddyt, hipStream_t s) {
  const int64_t Kg = F / M * 4;   // gathered columns
  if (dYt)
    return run_sddmm_dma<128, 512, 2, 4, 2, true, SD_VNM>(dY, lddy, Wd, ldw, Tn, Kg, Nc, hm, dz, dYt, lddyt, s, hc, V,
                                                           M, hv, relu, 0);
  return run_sddmm_dma<128, 512, 2, 4, 2, false, SD_VNM>(dY, lddy, Wd, ldw, Tn, Kg, Nc, hm, dz, nullptr, 0, s, hc, V,
                                                          M, hv, relu, 0);
}

// Dense NT GEMM out[r][c] = sum_t A[r][t] B[c][t] (fp32 out, row stride ldo), bf16 operands.
bool dense_nt_fast_ok(const void* A, int64_t lda, const void* B, int64_t ldb, const float* out, int64_t ldo,
                      int64_t Tn) {
  return Tn % TK == 0 && lda % 8 == 0 && ldb % 8 == 0 && ldo % 4 == 0 && (uintptr_t)A % 16 == 0 &&
         (uintptr_t)B % 16 == 0 && (uintptr_t)out % 16 == 0;
}

hipError_t launch_dense_nt(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t R, int64_t Kc, int64_t Tn,
                           float* out, int64_t ldo, hipStream_t s) {
  if (sd_w4_ok(R, lda, Kc, ldb, Tn))
    return run_sddmm_w4<false, SD_DENSE>(A, lda, B, ldb, R, Kc, Tn, nullptr, out, nullptr, 0, ldo, s);
  return run_sddmm_dma<256, 256, 4, 2, 2, false, SD_DENSE>(A, lda, B, ldb, R, Kc, Tn, nullptr, out, nullptr, 0, s,
                                                           nullptr, 1, 4, nullptr, 0, ldo);
}

}  // namespace nms
