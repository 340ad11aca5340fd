// Pipelined SpMM for 2:4 and V:N:M operands on gfx950 with
// v_smfmac_f32_32x32x32_bf16.
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
//  * global_load_lds_dwordx4 writes lane l's 16 bytes to M0 + 16*l.
//  * LDS read throughput per CU: ds_read_b128 ~2.6x ds_read_b64_tr_b16, so
//    the B operand is transposed in registers on its way into LDS and read
//    back with ds_read_b128.
//
// Data flow per workgroup (BM x BN tile of C, 64 dense k per step):
//  * values: direct-to-LDS, two steps (128 bytes of every row) at a time, as
//    whole rows, the 16-byte chunks of a row XOR-swizzled (apos) so that the
//    A operand reads -- one ds_read_b128 per fragment and 32-k half -- hit 16
//    distinct bank groups per 16 lanes;
//  * metadata: direct-to-LDS, 16 bytes per row and super-stage; one ds_read_b64
//    per fragment and step gives the index operands of both 32-k halves;
//  * B: each lane loads 8 rows x 8 columns (16-byte row loads, coalesced along
//    n; for V:N:M the 8 rows are two groups' selected rows), transposes them in
//    registers with v_perm and writes 16-byte k-runs to LDS laid out n-major
//    ([BN][64 k]), chunks XOR-swizzled by row (bpos); half of the lanes write
//    their columns in swapped pairs, so that both the writes and the
//    ds_read_b128 operand reads are free of bank conflicts;
//  * two LDS buffers for B, two A super-stages, and two register sets for B:
//    the B loads of steps k+1 and k+2 are in flight while step k runs on the
//    matrix cores; B of step k+1 is written to LDS after step k's instructions.
//    Tiles: 2:4 256 x 256 with one wave per SIMD (128 x 128 per wave,
//    accumulators in AGPRs); V:N:M with V % 128 == 0 128 x 256, one wave per
//    SIMD; other V:N:M 64 x 512 with two waves per SIMD (64 x 64 per wave): a
//    64-row block reuses each gathered B row only 64 times, so the L2 -> LDS
//    stream per matrix instruction is large, and the second wave per SIMD
//    keeps more LDS reads and loads in flight (19% faster at 2048 x 8192 x 4096,
//    V=64, than 64 x 256 with one wave per SIMD).
//    All loads are issued from inline assembly and waited for with explicit
//    vmcnt counts.
// Epilogue: each (fragment, element) store covers 128 contiguous bytes of a
// row of C (non-temporal: C is written once).
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {

// B rows are loaded with inline-assembly loads as well (load16_async, dma.hpp): their completion
// is counted by the same explicit vmcnt waits as the direct loads, and the wait takes the
// destination registers as in/out operands, so nothing reads them before the data has arrived.

// Swizzled 16-byte chunk position of chunk c in B row n (the LDS row of tile column n).  Chosen
// by measurement on gfx950: with it, 16 consecutive rows read at one chunk index, and the
// transposing writes (16 lanes writing columns 8b + (e ^ ((b >> 3) & 1)) of consecutive blocks
// b at one chunk), are both free of LDS bank conflicts.
__device__ __forceinline__ int bpos(int n, int chunk) { return chunk ^ (((n >> 1) ^ (n >> 4)) & 7); }

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct SpCfg {
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  // A super-stage = two 64-k steps: 64 kept bf16 (128 bytes) and 16 metadata bytes per row
  static constexpr int AV_BYTES = BM * 128;
  static constexpr int AM_BYTES = BM * 16;
  static constexpr int A_STAGE = AV_BYTES + AM_BYTES;
  static constexpr int B_STAGE = BN * 128;          // 64 k x 2 bytes per column
  static constexpr int LDS = 2 * A_STAGE + 2 * B_STAGE;
  static constexpr int AV_INSTR = AV_BYTES / 1024 / NW;   // 1 KB (8 rows) per direct load
  static constexpr int AM_LANES = BM / NW;               // one 16-byte metadata row per lane
  static constexpr int B_ROWS = 8;                      // each lane: 8 k rows x 8 columns of B per step
  static constexpr int L_A = AV_INSTR + 1;               // vmcnt of a super-stage's direct loads
  static constexpr int L_B = B_ROWS;                     // vmcnt of a step's B row loads
  static_assert(AV_BYTES % (1024 * NW) == 0 && AV_INSTR >= 1, "A blocks per wave");
  static_assert(AM_LANES >= 1 && AM_LANES <= 64 && BM % NW == 0, "metadata lanes per wave");
  static_assert(BN == NT, "one (8 k x 8 column) B block per lane: 8 chunks x BN/8 column blocks");
  static_assert(WM % 32 == 0 && WN % 32 == 0 && FM >= 1 && FN >= 1, "fragments");
  static_assert(L_A + L_B <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(NW == 4 || NW == 8, "a wave's B blocks: two 8-k chunks (lanes 0-31, 32-63) of 32 column blocks");
};

// 16-byte chunk position of chunk c in A row r (rows are 128 bytes = 8 chunks).  The two rows
// of a 256-byte LDS line share one XOR, consecutive lines take distinct ones: with this choice
// (measured on gfx950) 16 consecutive rows read at one chunk index are free of bank conflicts.
__device__ __forceinline__ int apos(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VENOM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void spmm_dma_kernel(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, const uint8_t* __restrict__ colsel,
    int64_t R, int64_t Kd, int V, int M, int64_t G, const uint16_t* __restrict__ B, int64_t ldb, int64_t Nc,
    float* __restrict__ C, int64_t ldc) {
  using Cfg = SpCfg<BM, BN, WAVES_M, WAVES_N>;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  extern __shared__ __align__(1024) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // tile coordinates: XCD-aware.  Grouped along M, except for V:N:M with 64-row tiles, which are
  // dealt column-panel-major (each XCD gathers the B rows of its own column panels only; every
  // V-row block selects a different half of B's rows, so row-grouped 64-row tiles pull nearly all
  // of B into every XCD's L2: 104 -> 95 us at 2048 x 8192 x 4096, V = 64).  The 128-row tiles keep
  // the grouped order (585 us against 655 column-panel-major at 8192 x 16384 x 4096, V = 128).
  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Nc + BN - 1) / BN);
  int tm, tn;
  if constexpr (VENOM && BM == 64) {
    panel_major_tile(blockIdx.x, ntm, ntn, 16, tm, tn);
  } else {
    const int nwg = ntm * ntn;
    const int wg = xcd_remap(blockIdx.x, nwg);
    constexpr int GM = 4;
    const int grp = wg / (GM * ntn);
    const int first_m = grp * GM;
    const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
    const int within = wg - grp * GM * ntn;
    tm = first_m + within % gsz;
    tn = within / gsz;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t vrow = Kd / 2;     // values per row
  const int64_t mrow = Kd / 8;     // metadata bytes per row
  const int KT = (int)(Kd / 64);   // 64-k steps (even: Kd % 128 == 0)
  const int64_t vblk = VENOM ? m0 / V : 0;
  const uint32_t smem_base = lds_addr(smem);
  unsigned char* const a_lds = smem;                          // 2 A super-stages
  unsigned char* const b_lds = smem + 2 * Cfg::A_STAGE;       // 2 B steps

  // ---- direct-load sources of a super-stage ----
  // values: instruction q covers rows 8q..8q+7; lane -> row 8q + lane/8, LDS chunk lane%8 holding
  // the row's 16-byte chunk (lane%8) ^ (row & 7)
  const uint16_t* a_src[Cfg::AV_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::AV_INSTR; ++t) {
    const int r = 8 * (wave * Cfg::AV_INSTR + t) + (lane >> 3);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    a_src[t] = values + row * vrow + 8 * apos(r, lane & 7);
  }
  // metadata: lane l < AM_LANES of wave w loads the 16 bytes of row w*AM_LANES + l
  const uint8_t* m_src;
  {
    int64_t row = m0 + wave * Cfg::AM_LANES + (lane < Cfg::AM_LANES ? lane : 0);
    row = row < R ? row : R - 1;
    m_src = meta + row * mrow;
  }
  // super-stage j (k-steps 2j, 2j+1) into A buffer `buf`
  auto issue_a = [&](int buf, int j) {
    const uint32_t st = smem_base + buf * Cfg::A_STAGE;
#pragma unroll
    for (int t = 0; t < Cfg::AV_INSTR; ++t)
      dma16(a_src[t] + (int64_t)j * 64, uniform(st + (wave * Cfg::AV_INSTR + t) * 1024));
    const uint32_t dst = uniform(st + Cfg::AV_BYTES + wave * Cfg::AM_LANES * 16);
    if constexpr (Cfg::AM_LANES == 64)
      dma16(m_src + (int64_t)j * 16, dst);
    else
      dma16_lanes(m_src + (int64_t)j * 16, dst, (1ull << Cfg::AM_LANES) - 1);
  };

  // ---- B: lane l of wave w owns k chunk bc = 2(w%4) + l/32 (k = 8bc .. 8bc+7 of the step) and
  //      column block bcb = l%32 + 32(w/4) (columns 8bcb .. 8bcb+7 of the tile) ----
  const int bc = 2 * (wave & 3) + (lane >> 5);
  const int bcb = (lane & 31) + 32 * (wave >> 2);
  int64_t b_col = n0 + 8 * bcb;
  b_col = b_col < Nc ? b_col : 0;          // columns past Nc: any valid data, never stored

  auto load_b = [&](int kt, u32x4 (&rb)[8]) {
    const int64_t k0 = (int64_t)kt * 64;
    int64_t rows[8];
    if constexpr (VENOM) {
      // 16 groups per step; the wave's lanes cover groups 4(w%4) .. 4(w%4)+3 (two per chunk): one
      // wave-uniform (scalar) load of their 16 column bytes.  k0 + 64 <= Kd, so all 16 exist.
      const int64_t g_first = (k0 >> 2) + 4 * (wave & 3);
      const u32x4 sel4 = *reinterpret_cast<const u32x4*>(colsel + 4 * (vblk * G + g_first));
      const uint32_t s_lo = (lane >> 5) ? sel4[2] : sel4[0];
      const uint32_t s_hi = (lane >> 5) ? sel4[3] : sel4[1];
      const int64_t g = g_first + 2 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rows[q] = g * M + ((s_lo >> (8 * q)) & (uint32_t)(M - 1));
        rows[q + 4] = (g + 1) * M + ((s_hi >> (8 * q)) & (uint32_t)(M - 1));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) rows[q] = k0 + 8 * bc + q;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) rb[q] = load16_async(B + rows[q] * ldb + b_col);
  };

  // B rows of a step, transposed, into B buffer `buf` ([BN][64 k], 16-byte chunks swizzled by bpos).
  // Write slot e stores one column's 8 k values (chunk bc) with one ds_write_b128; lanes with
  // bit 3 set write column e^1 in slot e, so every 16 lanes of a write cover both column parities
  // and 16 distinct bank groups.  v_perm picks the even or odd bf16 of each row pair.
  const int bflip = (lane >> 3) & 1;
  const uint32_t sel_lo = 0x05040100u, sel_hi = 0x07060302u;
  const uint32_t sel_even = bflip ? sel_hi : sel_lo, sel_odd = bflip ? sel_lo : sel_hi;
  auto store_b = [&](int buf, const u32x4 (&rb)[8]) {
    unsigned char* Bs = b_lds + buf * Cfg::B_STAGE;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = e >> 1;
      const uint32_t sel = (e & 1) ? sel_odd : sel_even;
      u32x4 d;
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = __builtin_amdgcn_perm(rb[2 * j + 1][p], rb[2 * j][p], sel);
      const int n = 8 * bcb + (e ^ bflip);
      *reinterpret_cast<u32x4*>(Bs + n * 128 + (bpos(n, bc) << 4)) = d;
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31, aa = lane >> 5;
  // Step kt: A super-stage buffer (kt/2)%2, half s = kt%2; B buffer kt%2.  The B rows of step kt+1
  // (register set rbs, waited for by `wait`) are transposed into B buffer (kt+1)%2 while the
  // matrix instructions of step kt run: the first half's operands are read first, the second
  // half's during the first half's 16 instructions, the transposes during the second half's.
  auto step = [&](int kt, const u32x4 (&rbs)[8], auto wait) {
    const int s = kt & 1;
    const unsigned char* As = a_lds + ((kt >> 1) & 1) * Cfg::A_STAGE;
    const unsigned char* Ms = As + Cfg::AV_BYTES;
    const unsigned char* Bs = b_lds + (kt & 1) * Cfg::B_STAGE;
    u32x2 mm[FM];
    uint32_t idx[2][FM];
    bf16x8 a[2][FM];
    bf16x16 b[2][FN];
    auto operands = [&](int h) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = (wm * FM + i) * 32 + l32;
        idx[h][i] = mm[i][h] >> (16 * aa);
        a[h][i] = *reinterpret_cast<const bf16x8*>(As + r * 128 + (apos(r, 4 * s + 2 * h + aa) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * Cfg::WN + 32 * j + l32;
        const unsigned char* row = Bs + n * 128;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(row + (bpos(n, 4 * h + aa) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(row + (bpos(n, 4 * h + 2 + aa) << 4));
        b[h][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
    };
    auto mfma = [&](int h) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[h][i], b[h][j], acc[i][j], (int)idx[h][i], 0, 0);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) mm[i] = *reinterpret_cast<const u32x2*>(Ms + ((wm * FM + i) * 32 + l32) * 16 + 8 * s);
    // the first half's operand reads are issued before anything else of the step (the scheduler
    // would otherwise sink them next to their matrix instructions and expose the LDS latency)
    operands(0);
    __builtin_amdgcn_sched_barrier(0);
    wait();
    operands(1);
    mfma(0);
    __builtin_amdgcn_sched_barrier(0);
    store_b((kt + 1) & 1, rbs);
    mfma(1);
  };

  // ---- pipeline ----
  // Even step kt = 2j: load the B rows of step kt+2, issue super-stage j+1 (k-steps kt+2, kt+3)
  // into the other A buffer, wait until only these loads are outstanding (so B of step kt+1 has
  // landed) and run step kt.  Odd step: load B of step kt+2, wait for everything but these loads
  // -- which includes super-stage j+1 -- and run step kt.  Loads complete in issue order.  Past
  // the end, loads repeat the last step / super-stage into buffers that are never read again,
  // so every step looks alike.
  const int klast = KT - 1, jlast = KT / 2 - 1;
  auto kc = [&](int k) { return k < klast ? k : klast; };
  u32x4 rb0[8], rb1[8];
  issue_a(0, 0);
  load_b(0, rb0);
  load_b(kc(1), rb1);
  wait_vmcnt_regs<Cfg::L_B>(rb0);     // super-stage 0 and B of step 0 have landed
  store_b(0, rb0);
  for (int kt = 0; kt < KT; kt += 2) {
    const int j = kt >> 1;
    // even step kt
    lds_barrier();   // step kt's A and B are in LDS for every wave; every wave is done with step kt-1
    load_b(kc(kt + 2), rb0);
    issue_a((j + 1) & 1, j + 1 < jlast ? j + 1 : jlast);
    step(kt, rb1, [&]() { wait_vmcnt_regs<Cfg::L_B + Cfg::L_A>(rb1); });
    // odd step kt+1
    lds_barrier();
    load_b(kc(kt + 3), rb1);
    step(kt + 1, rb0, [&]() { wait_vmcnt_regs<Cfg::L_B>(rb0); });
  }
  // Drain: no load may land in LDS or in a register after this point.  Both
  // register sets are operands of the wait, so neither can be reused before
  // its (redundant) loads have arrived.
  wait_vmcnt_regs<0>(rb0, rb1);

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

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VENOM>
static hipError_t run_dma(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t Kd,
                          int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                          hipStream_t s) {
  using Cfg = SpCfg<BM, BN, WAVES_M, WAVES_N>;
  const size_t lds = (size_t)Cfg::LDS;
  auto kern = spmm_dma_kernel<BM, BN, WAVES_M, WAVES_N, VENOM>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Nc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), lds, s, (const uint16_t*)values, meta, colsel, R,
                     Kd, V, M, G, (const uint16_t*)B, ldb, Nc, C, ldc);
  return hipGetLastError();
}

// Conditions: bf16, whole 128-k super-stages, 16-byte loads of values,
// metadata (16 bytes per row and super-stage) and B rows.
bool spmm_dma_ok(const void* values, const uint8_t* meta, const void* B, int64_t ldb, int64_t Nc, int64_t Kd) {
  return Kd % 128 == 0 && Kd >= 128 && Nc % 8 == 0 && ldb % 8 == 0 && (uintptr_t)values % 16 == 0 &&
         (uintptr_t)meta % 16 == 0 && (uintptr_t)B % 16 == 0;
}

hipError_t launch_spmm_nm_dma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                              int64_t ldb, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  return run_dma<256, 256, 2, 2, false>(values, meta, nullptr, R, K, 4, 4, K / 4, B, ldb, Nc, C, ldc, s);
}

hipError_t launch_spmm_venom_dma(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                                 int64_t Kd, int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc,
                                 float* C, int64_t ldc, hipStream_t s) {
  if (V % 128 == 0)
    return run_dma<128, 256, 1, 4, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
  return run_dma<64, 512, 1, 8, true>(values, meta, colsel, R, Kd, V, M, G, B, ldb, Nc, C, ldc, s);
}

}  // namespace nms
