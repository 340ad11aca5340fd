// Sparse x dense products C = A_sparse * B for the 2:4 and V:N:M formats (gfx950).
//
// "Success story: ESPLAG" (Research Topic, Solution) pairs the N:M / VENOM
// formats with an SpMM library; "To 2:4 Sparsity and Beyond" (abstract) runs
// every FFN matmul with a 2:4 weight or a v:n:m activation.  The product is
// the plain C[r][n] = sum_k A[r][k] B[k][n] with A given in compressed form.
//
// Fast path (bf16): the structured-sparse matrix instruction
// v_smfmac_f32_16x16x64_bf16 consumes the compressed values directly.  Its
// operand layout on gfx950 (established with a one-instruction probe):
//   A: lane l holds row l%16, the 8 kept values of dense k 16*(l/16)..+15;
//      the index operand holds, in its low 16 bits, one nibble p0 | p1 << 2
//      per group of 4, group 0 lowest -- exactly the stored 2:4 metadata, so
//      two bytes of a row's metadata go straight into the instruction;
//   B: lane l holds column l%16, k = 8*(l/16)..+7 in elements 0..7 and
//      k = 32 + 8*(l/16)..+7 in elements 8..15;
//   C: lane l holds column l%16, rows 4*(l/16)..+3.
// A V:N:M operand is a 2:4 operand over its selected columns: the selected
// rows of B are gathered (per V-row block, through colsel) while B is staged
// into LDS, after which the same inner loop runs.
//
// Data movement per workgroup and k-step (64 dense k of the 2:4 domain):
//   values [BM x 32] and metadata [BM x 8 bytes] -> LDS (row-major, padded);
//   B [64 x BN] is read with 16-byte row loads (n contiguous in HBM),
//   transposed in registers and written to LDS n-major (k contiguous), the
//   layout the B operand wants; LDS rows are permuted so that the 16 lanes
//   of one fragment read 16 consecutive LDS rows (no bank conflicts);
//   two LDS buffers, one barrier per k-step, global loads of step k+1 in
//   flight during the matrix instructions of step k.
// Fragment j of every 64-column group maps lane c to column 4c + j, so each
// lane ends up owning 4 consecutive columns of 4 rows and the epilogue writes
// 16-byte float4 stores that cover 256 contiguous bytes per row and wave.
#include "common.hpp"
#include "launch.hpp"

namespace nms {

// ---------------------------------------------------------------------------
// generic path: fp32 or bf16, any K % 4 == 0 (2:4) or V:N:M, any alignment.
// 64 x 64 tile, 256 lanes, 4 x 4 outputs per lane, A decompressed into LDS.
// ---------------------------------------------------------------------------
template <typename T, bool VENOM, typename OutT>
__global__ __launch_bounds__(256) void spmm_generic_kernel(const T* __restrict__ values, const uint8_t* __restrict__ meta,
                                                           const uint8_t* __restrict__ colsel, int64_t R, int64_t K,
                                                           int V, int M, const T* __restrict__ B, int64_t sbk,
                                                           int64_t sbn, int64_t Nc, OutT* __restrict__ C,
                                                           int64_t ldc) {
  constexpr int TM = 64, TN = 64, KC = 32;
  __shared__ float As[KC][TM + 4];
  __shared__ float Bs[KC][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int Mg = VENOM ? M : 4;                 // dense width of a group
  const int64_t G = K / Mg;                     // groups per row
  const int64_t vrow = G * 2;                   // values per row
  const int64_t mrow = (G + 1) / 2;             // metadata bytes per row
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    // A: zero, then scatter the kept values of each (row, group) unit
    for (int i = tid; i < KC * TM; i += 256) As[i / TM][i % TM] = 0.f;
    __syncthreads();
    const int gpc = KC / Mg;                    // groups per chunk
    for (int u = tid; u < TM * gpc; u += 256) {
      const int r = u / gpc, gi = u % gpc;
      const int64_t row = m0 + r, g = k0 / Mg + gi;
      if (row >= R || g >= G) continue;
      const uint32_t nib = (meta[row * mrow + g / 2] >> (4 * (g & 1))) & 0xF;
      for (int s = 0; s < 2; ++s) {
        const uint32_t p = (nib >> (2 * s)) & 3;
        const uint32_t col = VENOM ? (colsel[((row / V) * G + g) * 4 + p] & (uint32_t)(Mg - 1)) : p;
        As[gi * Mg + col][r] = Elem<T>::to_f32(values[row * vrow + 2 * g + s]);
      }
    }
    for (int i = tid; i < KC * TN; i += 256) {
      const int kk = i / TN, nn = i % TN;
      const int64_t k = k0 + kk, n = n0 + nn;
      Bs[kk][nn] = (k < K && n < Nc) ? Elem<T>::to_f32(B[k * sbk + n * sbn]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= R) continue;
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < Nc) store_out(C + row * ldc + n, acc[i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: v_mfma_f32_16x16x4f32 on the decompressed operand.  There is no
// structured-sparse fp32 matrix instruction, so the 2:4 rows are expanded (two
// kept values and two +0.0 per group) into LDS.  A workgroup owns a 16 x 16
// tile of C and stages up to 256 k of A (16 rows) and B (16 columns) at once;
// its four waves take interleaved 4-k steps (wave w: steps w, w+4, ...) with
// one matrix instruction each, and wave 0 adds the four partial tiles in wave
// order (a fixed summation order: the result does not depend on timing).
// v_mfma_f32_16x16x4f32: lane l holds A[row l%16][k l/16] and B[k l/16][col
// l%16]; the result holds column l%16, rows 4*(l/16) .. +3.
// ---------------------------------------------------------------------------
constexpr int F32_KC = 256;   // k staged per chunk (38 KB of LDS)

__global__ __launch_bounds__(256) void spmm_f32_mfma_kernel(const float* __restrict__ values,
                                                            const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                            const float* __restrict__ B, int64_t sbk, int64_t sbn,
                                                            int64_t Nc, float* __restrict__ C, int64_t ldc) {
  __shared__ float As[16][F32_KC + 4];
  __shared__ float Bs[F32_KC][16 + 1];
  __shared__ f32x4 part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * 16, n0 = (int64_t)blockIdx.x * 16;
  const int64_t G = K / 4, vrow = K / 2, mrow = (G + 1) / 2;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < K; k0 += F32_KC) {
    const int kc = (int)((K - k0) < F32_KC ? (K - k0) : F32_KC);   // a multiple of 4
    // A: one (row, group) unit per thread and pass: both kept values and the two zeros
    for (int u = tid; u < 16 * (kc / 4); u += 256) {
      const int r = u / (kc / 4), gi = u % (kc / 4);
      const int64_t row = m0 + r, g = k0 / 4 + gi;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
      if (row < R) {
        const uint32_t nib = (meta[row * mrow + g / 2] >> (4 * (g & 1))) & 0xF;
        a4[nib & 3] = values[row * vrow + 2 * g];
        a4[(nib >> 2) & 3] = values[row * vrow + 2 * g + 1];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) As[r][4 * gi + p] = a4[p];
    }
    for (int i = tid; i < 16 * kc; i += 256) {
      const int kk = i / 16, nn = i % 16;
      const int64_t n = n0 + nn;
      Bs[kk][nn] = n < Nc ? B[(k0 + kk) * sbk + n * sbn] : 0.f;
    }
    __syncthreads();
    for (int st = wave; st < kc / 4; st += 4) {
      const int k = 4 * st + (lane >> 4);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(As[lane & 15][k], Bs[k][lane & 15], acc, 0, 0, 0);
    }
    __syncthreads();
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = part[w][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += o[e];
    }
    const int64_t col = n0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + 4 * (lane >> 4) + e;
      if (row < R && col < Nc) C[row * ldc + col] = sum[e];
    }
  }
}

static hipError_t run_f32_mfma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                               int64_t sbk, int64_t sbn, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  const dim3 grid((unsigned)((Nc + 15) / 16), (unsigned)((R + 15) / 16));
  hipLaunchKernelGGL(spmm_f32_mfma_kernel, grid, dim3(256), 0, s, (const float*)values, meta, R, K, (const float*)B,
                     sbk, sbn, Nc, C, ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fast path: bf16, v_smfmac_f32_16x16x64_bf16
// ---------------------------------------------------------------------------
constexpr int SK = 64;          // dense k (2:4 domain) per k-step
constexpr int A_PITCH = 40;     // u16 per LDS row of values: 32 + 8 pad (80 bytes)
constexpr int B_PITCH = 72;     // u16 per LDS row of B (one column n): 64 + 8 pad (144 bytes)

// LDS row of column n inside a tile: fragment j of a 64-column group reads
// columns 4c + j (c = 0..15); they are stored in rows 16j + c.
__device__ inline int b_lds_row(int n) { return (n & ~63) | ((n & 3) << 4) | ((n & 63) >> 2); }

template <int BM, int BN, int WM, int WN, bool VENOM>
struct SmfmacCfg {
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;           // fragments per wave
  static constexpr int A_CHUNKS = BM * 4 / NT;               // 16-byte value chunks per lane
  static constexpr int B_RB = SK * BN / 8 / NT;              // B rows per lane block (x 8 columns)
  static constexpr int B_BLOCKS_N = BN / 8;
  static constexpr int LDS_A = BM * A_PITCH * 2;             // bytes
  static constexpr int LDS_M = BM * 8;
  static constexpr int LDS_B = BN * B_PITCH * 2;
  static constexpr int STAGE = LDS_A + LDS_M + LDS_B;
  static_assert(WN % 64 == 0, "wave tile must hold whole 64-column groups");
  static_assert(BM * 4 % NT == 0 && BM <= NT, "A chunking");
  static_assert(B_RB == 4 || B_RB == 8, "B block rows");
  static_assert(NT == 256, "kernels are compiled for 256-lane workgroups");
};

template <int BM, int BN, int WM, int WN, bool VENOM>
__global__ __launch_bounds__(256) void spmm_smfmac_kernel(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, const uint8_t* __restrict__ colsel,
    int64_t R, int64_t Kd, int V, int M, int64_t G, const uint16_t* __restrict__ B, int64_t ldb, int64_t Nc,
    float* __restrict__ C, int64_t ldc) {
  using Cfg = SmfmacCfg<BM, BN, WM, WN, VENOM>;
  constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN, RB = Cfg::B_RB;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;

  // tile coordinates: XCD-aware, grouped along M so co-resident tiles share panels
  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Nc + BN - 1) / BN);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  constexpr int GM = 8;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t vrow = Kd / 2;          // values per row
  const int64_t mrow = (Kd + 7) / 8;    // metadata bytes per row
  const int64_t vblk = VENOM ? m0 / V : 0;
  const int KT = (int)((Kd + SK - 1) / SK);

  // ---- per-lane global load assignment ----
  // A values: chunk c = tid + i*NT -> row c/4, 16-byte part c%4
  // metadata: row tid (BM <= NT), 8 bytes as four u16
  // B: block (kb, nb): rows kb*RB..+RB-1, columns nb*8..+7
  const int b_nb = tid % Cfg::B_BLOCKS_N, b_kb = tid / Cfg::B_BLOCKS_N;

  u32x4 ra[Cfg::A_CHUNKS];
  uint16_t rm[4];
  u32x4 rb[RB];

  auto load_global = [&](int kt) {
    const int64_t k0 = (int64_t)kt * SK;
#pragma unroll
    for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 2, part = c & 3;
      const int64_t row = m0 + r, kk = k0 + part * 16;
      if (row < R && kk < Kd)
        ra[i] = *reinterpret_cast<const u32x4*>(values + row * vrow + kk / 2);
      else
        ra[i] = u32x4{0, 0, 0, 0};
    }
    if (tid < BM) {
      const int64_t row = m0 + tid;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t kk = k0 + q * 16;
        rm[q] = (row < R && kk < Kd) ? *reinterpret_cast<const uint16_t*>(meta + row * mrow + kk / 8) : (uint16_t)0;
      }
    }
    const int64_t n = n0 + b_nb * 8;
    uint32_t rsel = 0, rsel2 = 0;
    if constexpr (VENOM) {
      const int64_t kd = k0 + b_kb * RB;           // first 2:4-domain row of this block (multiple of 4)
      const int64_t g = kd / 4;
      if (g < G) rsel = *reinterpret_cast<const uint32_t*>(colsel + (vblk * G + g) * 4);
      if (RB == 8 && g + 1 < G) rsel2 = *reinterpret_cast<const uint32_t*>(colsel + (vblk * G + g + 1) * 4);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int64_t kd = k0 + b_kb * RB + i;
      int64_t krow = kd;
      if constexpr (VENOM) {
        const uint32_t sel = (i < 4) ? rsel : rsel2;
        krow = (kd >> 2) * M + ((sel >> (8 * (i & 3))) & (uint32_t)(M - 1));
      }
      if (kd < Kd && n < Nc)
        rb[i] = *reinterpret_cast<const u32x4*>(B + krow * ldb + n);
      else
        rb[i] = u32x4{0, 0, 0, 0};
    }
  };

  auto store_lds = [&](int buf) {
    unsigned char* st = smem + buf * Cfg::STAGE;
    uint16_t* As = reinterpret_cast<uint16_t*>(st);
    uint8_t* Ms = st + Cfg::LDS_A;
    uint16_t* Bs = reinterpret_cast<uint16_t*>(st + Cfg::LDS_A + Cfg::LDS_M);
#pragma unroll
    for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      const int r = c >> 2, part = c & 3;
      *reinterpret_cast<u32x4*>(As + r * A_PITCH + part * 8) = ra[i];
    }
    if (tid < BM) {
      uint32_t lo = (uint32_t)rm[0] | ((uint32_t)rm[1] << 16), hi = (uint32_t)rm[2] | ((uint32_t)rm[3] << 16);
      *reinterpret_cast<u32x2*>(Ms + tid * 8) = u32x2{lo, hi};
    }
    // transpose the RB x 8 block: column e gets RB consecutive k values
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t w[RB / 2];
#pragma unroll
      for (int i = 0; i < RB / 2; ++i) {
        const uint32_t x0 = rb[2 * i][e >> 1], x1 = rb[2 * i + 1][e >> 1];
        // low half = column e of row 2i, high half = column e of row 2i+1
        w[i] = (e & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
      }
      const int lr = b_lds_row(b_nb * 8 + e);
      uint16_t* dst = Bs + lr * B_PITCH + b_kb * RB;
      if constexpr (RB == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      } else {
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
      }
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
    const uint8_t* Ms = st + Cfg::LDS_A;
    const uint16_t* Bs = reinterpret_cast<const uint16_t*>(st + Cfg::LDS_A + Cfg::LDS_M);
    bf16x8 a[FM];
    int idx[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + i * 16 + lr16;
      a[i] = *reinterpret_cast<const bf16x8*>(As + r * A_PITCH + lg * 8);
      idx[i] = (int)*reinterpret_cast<const uint16_t*>(Ms + r * 8 + lg * 2);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int lrow = wn * WN + (f >> 2) * 64 + (f & 3) * 16 + lr16;
      const uint16_t* bp = Bs + lrow * B_PITCH + lg * 8;
      const bf16x8 lo = *reinterpret_cast<const bf16x8*>(bp);
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(bp + 32);
      const bf16x16 b = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][f] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a[i], b, acc[i][f], idx[i], 0, 0);
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

  // epilogue: fragment (i, f = 4*grp + j), element e -> row 16i + 4*lg + e,
  // column 64*grp + 4*lr16 + j
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + wm * WM + i * 16 + lg * 4 + e;
#pragma unroll
      for (int grp4 = 0; grp4 < FN / 4; ++grp4) {
        const int64_t col = n0 + wn * WN + grp4 * 64 + lr16 * 4;
        if (row < R && col < Nc) {
          f32x4 o = {acc[i][grp4 * 4 + 0][e], acc[i][grp4 * 4 + 1][e], acc[i][grp4 * 4 + 2][e], acc[i][grp4 * 4 + 3][e]};
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(C + row * ldc + col));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool VENOM>
static hipError_t run_smfmac(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t Kd,
                             int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                             hipStream_t s) {
  using Cfg = SmfmacCfg<BM, BN, WM, WN, VENOM>;
  const size_t lds = 2 * (size_t)Cfg::STAGE;
  auto kern = spmm_smfmac_kernel<BM, BN, WM, WN, VENOM>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Nc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), lds, s, (const uint16_t*)values, meta, colsel, R,
                     Kd, V, M, G, (const uint16_t*)B, ldb, Nc, C, ldc);
  return hipGetLastError();
}

template <typename T, bool VENOM, typename OutT>
static hipError_t run_generic(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t K,
                              int V, int M, const void* B, int64_t sbk, int64_t sbn, int64_t Nc, OutT* C, int64_t ldc,
                              hipStream_t s) {
  dim3 grid((unsigned)((Nc + 63) / 64), (unsigned)((R + 63) / 64));
  hipLaunchKernelGGL((spmm_generic_kernel<T, VENOM, OutT>), grid, dim3(256), 0, s, (const T*)values, meta, colsel, R,
                     K, V, M, (const T*)B, sbk, sbn, Nc, C, ldc);
  return hipGetLastError();
}

// Conditions of the SMFMAC path: 16-byte vector loads of values and B rows,
// 2-byte metadata loads, 16-byte float4 stores of C.
static bool fast_ok(const void* values, const uint8_t* meta, const void* B, int64_t ldb, int64_t Nc, const float* C,
                    int64_t ldc, int64_t Kd) {
  return Kd % 16 == 0 && Nc % 8 == 0 && ldb % 8 == 0 && ldc % 4 == 0 && (uintptr_t)values % 16 == 0 &&
         (uintptr_t)meta % 2 == 0 && (uintptr_t)B % 16 == 0 && (uintptr_t)C % 16 == 0;
}

// Kernel selection knob, read on every call (for A/B tests of the tiers):
// NMSPARSE_SPMM_TIER=1 skips the pipelined DMA kernel (register-staged SMFMAC
// kernel instead); NMSPARSE_SPMM_TIER=2 skips the register-gather V:N:M kernel
// (the pipelined DMA kernel instead); NMSPARSE_FORCE_GENERIC (common.hpp)
// selects the SIMT kernel.
static int kernel_tier() {
  const char* e = getenv("NMSPARSE_SPMM_TIER");
  return e && (e[0] == '1' || e[0] == '2') ? e[0] - '0' : 0;
}

hipError_t launch_spmm_nm(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                          int64_t ldb, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  if (dt == DT_BF16 && !force_generic() && kernel_tier() == 0 && spmm_dma_ok(values, meta, B, ldb, Nc, K))
    return launch_spmm_nm_dma(values, meta, R, K, B, ldb, Nc, C, ldc, s);
  if (dt == DT_BF16 && !force_generic() && fast_ok(values, meta, B, ldb, Nc, C, ldc, K))
    return run_smfmac<256, 128, 128, 64, false>(values, meta, nullptr, R, K, 4, 4, K / 4, B, ldb, Nc, C, ldc, s);
  if (dt == DT_F32 && !force_generic()) return run_f32_mfma(values, meta, R, K, B, ldb, 1, Nc, C, ldc, s);
  return dt == DT_BF16 ? run_generic<uint16_t, false>(values, meta, nullptr, R, K, 4, 4, B, ldb, 1, Nc, C, ldc, s)
                       : run_generic<uint32_t, false>(values, meta, nullptr, R, K, 4, 4, B, ldb, 1, Nc, C, ldc, s);
}

hipError_t launch_spmm_nm_t(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                            int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  if (dt == DT_BF16 && !force_generic() && spmm_nt_ok(values, meta, Bt, ldbt, R, Nc, K))
    return launch_spmm_nm_nt_dma(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
  if (dt == DT_F32 && !force_generic()) return run_f32_mfma(values, meta, R, K, Bt, 1, ldbt, Nc, C, ldc, s);
  return dt == DT_BF16 ? run_generic<uint16_t, false>(values, meta, nullptr, R, K, 4, 4, Bt, 1, ldbt, Nc, C, ldc, s)
                       : run_generic<uint32_t, false>(values, meta, nullptr, R, K, 4, 4, Bt, 1, ldbt, Nc, C, ldc, s);
}

hipError_t launch_spmm_nm_t_bf16out(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                   const void* Bt, int64_t ldbt, int64_t Nc, uint16_t* C, int64_t ldc, hipStream_t s) {
  if (dt == DT_BF16 && !force_generic() && spmm_nt_ok(values, meta, Bt, ldbt, R, Nc, K))
    return launch_spmm_nm_nt_dma_bf16out(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
  return dt == DT_BF16 ? run_generic<uint16_t, false>(values, meta, nullptr, R, K, 4, 4, Bt, 1, ldbt, Nc, C, ldc, s)
                       : run_generic<uint32_t, false>(values, meta, nullptr, R, K, 4, 4, Bt, 1, ldbt, Nc, C, ldc, s);
}

hipError_t launch_spmm_venom(int dt, const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                             int64_t K, int V, int M, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                             hipStream_t s) {
  const int64_t G = K / M;
  const int64_t Kd = G * 4;  // the 2:4 domain: 4 selected columns per group
  if (dt == DT_BF16 && !force_generic() && kernel_tier() == 0 && spmm_dma_ok(values, meta, B, ldb, Nc, Kd) &&
      spmm_vnm_reg_ok(colsel, V, M, G, Kd, ldb, Nc, C, ldc))
    return launch_spmm_vnm_reg(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
  if (dt == DT_BF16 && !force_generic() && kernel_tier() != 1 && spmm_dma_ok(values, meta, B, ldb, Nc, Kd) &&
      (uintptr_t)colsel % 16 == 0 && V % 64 == 0)
    return launch_spmm_venom_dma(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
  if (dt == DT_BF16 && !force_generic() && fast_ok(values, meta, B, ldb, Nc, C, ldc, Kd) &&
      (uintptr_t)colsel % 4 == 0) {
    if (V % 128 == 0)
      return run_smfmac<128, 256, 64, 128, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
    if (V % 64 == 0)
      return run_smfmac<64, 256, 64, 64, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
  }
  return dt == DT_BF16 ? run_generic<uint16_t, true>(values, meta, colsel, R, K, V, M, B, ldb, 1, Nc, C, ldc, s)
                       : run_generic<uint32_t, true>(values, meta, colsel, R, K, V, M, B, ldb, 1, Nc, C, ldc, s);
}

}  // namespace nms
