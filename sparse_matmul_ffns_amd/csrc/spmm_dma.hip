// Pipelined SpMM for 2:4 and V:N:M operands on gfx950: direct-to-LDS loads,
// transposing LDS reads and v_smfmac_f32_32x32x32_bf16.
//
// Product: C[r][n] = sum_k A[r][k] B[k][n], A in 2:4 form (values + nibbles),
// or V:N:M form, which is 2:4 over the selected columns with the selected rows
// of B gathered through colsel ("Success story: ESPLAG", Solution; "To 2:4
// Sparsity and Beyond", abstract).
//
// Layout facts of gfx950 used here (each measured with a one-off probe):
//  * v_smfmac_f32_32x32x32_bf16: lane l holds A row l%32 with the 8 kept
//    values of dense k 16*(l/32)..+15 (index operand: one nibble p0 | p1 << 2
//    per group of 4, group 0 in bits 0..3 -- the stored metadata order);
//    B column l%32 with k = 8*(l/32)..+7 in elements 0..7 and
//    k = 16 + 8*(l/32)..+7 in elements 8..15; C column l%32, element e at
//    row 8*(e/4) + 4*(l/32) + e%4.
//  * global_load_lds_dwordx4 writes lane l's 16 bytes to M0 + 16*l: a wave
//    fills 1 KB of LDS in lane order, from any 64 global addresses.
//  * ds_read_b64_tr_b16, per 16-lane group: with lane i addressing the 4
//    elements at row kb + i/4, columns c0 + 4*(i%4)..+3 of a row-major tile,
//    lane j receives B[kb + t][c0 + j] for t = 0..3 -- four consecutive k of
//    one column, i.e. the transposed operand.
//
// Data flow per workgroup (BM x BN tile of C, 64 dense k per stage):
//  * values: one 1 KB block per (32-row fragment, 32-k half), lanes in
//    instruction order, so every A operand read is one conflict-free
//    ds_read_b128 at block + 16*lane;
//  * metadata: [BM][8 bytes] row-major; one ds_read_b64 per 32-row fragment
//    yields the index operands of both k halves;
//  * B: [64][BN] row-major as stored in HBM (rows gathered through colsel
//    for V:N:M), 16-byte chunks XOR-swizzled per row so that the four rows a
//    16-lane group reads in one transposing read fall in distinct banks;
//  * STAGES-deep ring of LDS buffers; the loads of stage k+2 are in flight
//    while stage k runs on the matrix cores.  Loads are issued with inline
//    assembly and waited for with explicit vmcnt counts, so the compiler's
//    conservative waits for LDS DMA never serialise the pipeline.
// Epilogue: each (fragment, element) store covers 128 contiguous bytes of a
// row of C (non-temporal: C is written once).
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// swizzle of the 16-byte chunk index of B row r
__device__ __forceinline__ int bswz(int r) { return (r & 3) << 1; }

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
struct DmaCfg {
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * 64;                  // 32 kept bf16 per row and stage
  static constexpr int M_BYTES = BM * 8;
  static constexpr int B_ROW = BN * 2;                     // bytes per B row in LDS
  static constexpr int B_BYTES = 64 * B_ROW;
  static constexpr int STAGE = A_BYTES + M_BYTES + B_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / NW;      // per wave and stage
  static constexpr int M_LANES = M_BYTES / 4 / NW;          // one dword DMA per wave, M_LANES lanes active
  static constexpr int B_INSTR = B_BYTES / 1024 / NW;
  static constexpr int LOADS = A_INSTR + 1 + B_INSTR;      // vmcnt per stage per wave
  static_assert(A_BYTES % (1024 * NW) == 0, "A blocks per wave");
  static_assert(M_BYTES % (4 * NW) == 0 && M_LANES >= 1 && M_LANES <= 64, "metadata lanes per wave");
  static_assert(B_BYTES % (1024 * NW) == 0 && (B_ROW % 1024 == 0 || 1024 % B_ROW == 0), "B blocks per wave");
  static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "fragments");
  static_assert(LOADS * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(1024 % B_ROW != 0 || 1024 / B_ROW <= 4, "rows of one B DMA instruction share a group of 4");
  static_assert(STAGE * STAGES <= 160 * 1024, "LDS budget");
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool VENOM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void spmm_dma_kernel(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, const uint8_t* __restrict__ colsel,
    int64_t R, int64_t Kd, int V, int M, int64_t G, const uint16_t* __restrict__ B, int64_t ldb, int64_t Nc,
    float* __restrict__ C, int64_t ldc) {
  using Cfg = DmaCfg<BM, BN, WAVES_M, WAVES_N, STAGES>;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  extern __shared__ __align__(1024) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // tile coordinates: XCD-aware, grouped along M
  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Nc + BN - 1) / BN);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  constexpr int GM = 4;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t vrow = Kd / 2;     // values per row
  const int64_t mrow = Kd / 8;     // metadata bytes per row (Kd % 64 == 0)
  const int KT = (int)(Kd / 64);
  const int64_t vblk = VENOM ? m0 / V : 0;
  const uint32_t smem_base = lds_addr(smem);

  // ---- per-lane DMA sources that do not depend on the stage ----
  // A block q (q = wave*A_INSTR + t): 32-row fragment q/2, k half q%2; lane -> row 32*(q/2) + lane%32,
  // 16-byte chunk 2*(q%2) + lane/32 of the stage's 64 bytes
  const uint16_t* a_src[Cfg::A_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::A_INSTR; ++t) {
    const int q = wave * Cfg::A_INSTR + t;
    int64_t row = m0 + 32 * (q >> 1) + (lane & 31);
    row = row < R ? row : R - 1;
    a_src[t] = values + row * vrow + 8 * (2 * (q & 1) + (lane >> 5));
  }
  // metadata: wave w, lane l < M_LANES loads the dword at byte (w*M_LANES + l)*4 of the [BM][8] tile
  const uint8_t* m_src;
  {
    const int o = (wave * Cfg::M_LANES + (lane < Cfg::M_LANES ? lane : 0)) * 4;
    int64_t row = m0 + (o >> 3);
    row = row < R ? row : R - 1;
    m_src = meta + row * mrow + (o & 7);
  }
  // B: instruction q covers LDS bytes q*1024.. of the [64][BN] tile
  int b_row[Cfg::B_INSTR];
  int64_t b_col[Cfg::B_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::B_INSTR; ++t) {
    const int q = wave * Cfg::B_INSTR + t;
    const int byte = q * 1024 + lane * 16;
    const int r = byte / Cfg::B_ROW;
    const int p = (byte % Cfg::B_ROW) / 16;          // chunk position in the LDS row
    const int c = p ^ bswz(r);                         // global chunk held there
    int64_t col = n0 + 8 * c;
    col = col < Nc ? col : 0;                          // columns past Nc: any valid data, never stored
    b_row[t] = r;
    b_col[t] = col;
  }

  auto issue = [&](int kt) {
    const int buf = kt % STAGES;
    const uint32_t st = smem_base + buf * Cfg::STAGE;
    const int64_t k0 = (int64_t)kt * 64;
#pragma unroll
    for (int t = 0; t < Cfg::A_INSTR; ++t)
      dma16(a_src[t] + k0 / 2, uniform(st + (wave * Cfg::A_INSTR + t) * 1024));
    {
      // lanes >= M_LANES are masked off; the instruction still counts once in vmcnt
      const uint32_t dst = uniform(st + Cfg::A_BYTES + wave * Cfg::M_LANES * 4);
      if (Cfg::M_LANES == 64 || lane < Cfg::M_LANES) dma4(m_src + k0 / 8, dst);
    }
#pragma unroll
    for (int t = 0; t < Cfg::B_INSTR; ++t) {
      int64_t krow = k0 + b_row[t];
      if constexpr (VENOM) {
        // every row of one DMA instruction lies in the same group of 4 selected
        // columns, so the group's 4 column bytes are one wave-uniform (scalar) load
        const int q = wave * Cfg::B_INSTR + t;
        const int64_t g = (k0 + (q * 1024) / Cfg::B_ROW) >> 2;
        const uint32_t sel4 = reinterpret_cast<const uint32_t*>(colsel)[vblk * G + g];
        const uint32_t sel = (sel4 >> (8 * (krow & 3))) & (uint32_t)(M - 1);
        krow = g * M + sel;
      }
      dma16(B + krow * ldb + b_col[t], uniform(st + Cfg::A_BYTES + Cfg::M_BYTES + (wave * Cfg::B_INSTR + t) * 1024));
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // per-lane LDS read offsets that do not depend on the stage
  const int l32 = lane & 31, aa = lane >> 5;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int bb = g16 >> 1, half16 = g16 & 1;
  // B transposing read: lane addresses row (kbase + i16/4), columns cb + 16*half16 + 4*(i16%4)
  int b_off[FN][2][4];
  constexpr int KOFF[4] = {0, 4, 16, 20};
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int r = 32 * h + 8 * bb + KOFF[e4] + (i16 >> 2);
        const int cel = wn * Cfg::WN + 32 * j + 16 * half16 + 4 * (i16 & 3);
        const int c = cel >> 3;
        b_off[j][h][e4] = r * Cfg::B_ROW + ((c ^ bswz(r)) << 4) + ((cel & 7) << 1);
      }

  auto compute = [&](int kt) {
    const int buf = kt % STAGES;
    const unsigned char* st = smem + buf * Cfg::STAGE;
    const unsigned char* As = st;
    const unsigned char* Ms = st + Cfg::A_BYTES;
    const unsigned char* Bs = st + Cfg::A_BYTES + Cfg::M_BYTES;
    uint32_t idx[FM][2];
    bf16x8 a[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rf = wm * FM + i;  // 32-row fragment index within the tile
      const u32x2 mm = *reinterpret_cast<const u32x2*>(Ms + (rf * 32 + l32) * 8);
      idx[i][0] = aa ? (mm[0] >> 16) : mm[0];
      idx[i][1] = aa ? (mm[1] >> 16) : mm[1];
#pragma unroll
      for (int h = 0; h < 2; ++h) a[i][h] = *reinterpret_cast<const bf16x8*>(As + (rf * 2 + h) * 1024 + lane * 16);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Bs + b_off[j][h][0]));
        s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Bs + b_off[j][h][1]));
        s16x4 p2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Bs + b_off[j][h][2]));
        s16x4 p3 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Bs + b_off[j][h][3]));
        typedef short s16x16 __attribute__((ext_vector_type(16)));
        s16x16 bv = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7),
                                            __builtin_shufflevector(p2, p3, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5,
                                            6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        const bf16x16 b = __builtin_bit_cast(bf16x16, bv);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[i][h], b, acc[i][j], (int)idx[i][h], 0, 0);
      }
    }
  };

  // ---- pipeline ----
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    // own loads of stage kt have landed when at most (stages issued after it) remain
    if (kt + STAGES - 2 < KT) wait_vmcnt<Cfg::LOADS * (STAGES - 2)>();
    else wait_vmcnt<0>();
    barrier();   // every wave's stage-kt data is in LDS; every wave is done with stage kt-1
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);
    compute(kt);
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * Cfg::WN + 32 * j + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * Cfg::WM + 32 * i + 8 * (e >> 2) + 4 * aa + (e & 3);
        if (row < R && col < Nc) __builtin_nontemporal_store(acc[i][j][e], C + row * ldc + col);
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool VENOM>
static hipError_t run_dma(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t Kd,
                          int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                          hipStream_t s) {
  using Cfg = DmaCfg<BM, BN, WAVES_M, WAVES_N, STAGES>;
  const size_t lds = (size_t)Cfg::STAGE * STAGES;
  auto kern = spmm_dma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, VENOM>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Nc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), lds, s, (const uint16_t*)values, meta, colsel, R,
                     Kd, V, M, G, (const uint16_t*)B, ldb, Nc, C, ldc);
  return hipGetLastError();
}

// Conditions: bf16, 64-element k-steps without a tail, 16-byte loads of
// values and B rows, 4-byte metadata loads.
bool spmm_dma_ok(const void* values, const uint8_t* meta, const void* B, int64_t ldb, int64_t Nc, int64_t Kd) {
  return Kd % 64 == 0 && Kd >= 64 && Nc % 8 == 0 && ldb % 8 == 0 && (uintptr_t)values % 16 == 0 &&
         (uintptr_t)meta % 4 == 0 && (uintptr_t)B % 16 == 0;
}

hipError_t launch_spmm_nm_dma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                              int64_t ldb, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  return run_dma<256, 256, 2, 4, 3, false>(values, meta, nullptr, R, K, 4, 4, K / 4, B, ldb, Nc, C, ldc, s);
}

hipError_t launch_spmm_venom_dma(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                                 int64_t Kd, int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc,
                                 float* C, int64_t ldc, hipStream_t s) {
  if (V % 128 == 0)
    return run_dma<128, 256, 2, 4, 3, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
  return run_dma<64, 256, 1, 4, 3, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
}

}  // namespace nms
