// 2:4 SpMM on the panel layout of the compressed weight, four waves (gfx950).
//
// Product: C[r][n] = sum_k A[r][k] Bt[n][k], A in 2:4 form ("Success story: ESPLAG", Research
// Topic: the SpMM of a 2:4 layer; NSF PAR award 2340011, SLOPE abstract: the backward pass's
// product with the re-pruned transposed weight), Bt K-contiguous as for spmm_nm_t.
//
// The panel layout holds the values and nibbles of the row-major form in another order:
//   values: the 64 bytes of row r for the 64-column step s (its 32 kept values) at byte
//           ((r / 2) * (K / 64) + s) * 128 + (r % 2) * 64 -- one 128-byte line per row pair
//           and step;
//   meta:   the 32 bytes of row r for the 256-column chunk c (its 64 nibbles) at byte
//           ((r / 4) * (K / 256) + c) * 128 + (r % 4) * 32 -- one line per 4 rows and chunk;
// within a piece, the row-major order.  Each step of the kernel then reads whole lines of every
// operand (the vector L1 spends about two cycles per 128-byte line an instruction touches), which
// lets every operand be loaded two steps ahead through a ring of three LDS stages (160 KB)
// without reading half lines.
//
// Four waves of 128 x 128 (4 x 4 v_smfmac_f32_32x32x32_bf16 fragments, the 256 fp32 accumulators
// of a wave in the accumulation registers, one wave per SIMD) on a 256 x 256 tile.  A wave reads
// 0.75 KB of LDS per matrix instruction against 1 KB with eight waves of 128 x 64: the LDS reads
// and the matrix instructions are the two parts that each fill most of a step of the eight-wave
// kernel (spmm_nt.hip).  Every LDS read and load is issued between two matrix instructions, and
// the barrier sits between a step's two halves: the first half reads the step's second-half
// operands, the second half the next step's first-half operands and metadata, and loads the
// stage three steps ahead into the slot the barrier has just freed.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {

// largest C (bytes) written with ordinary stores (the rule of the eight-wave kernel)
constexpr int64_t kW4CachedCBytes = int64_t(160) << 20;

// XOR of the 16-byte chunk c (0..3) of row r in a values stage (rows in pairs per 128-byte line):
// the reads of 16 consecutive rows at one chunk, and of 8, fall on distinct 16-byte bank slots
__device__ __forceinline__ int pw_f(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int pw_apos(int r, int c) { return (r >> 1) * 128 + (r & 1) * 64 + ((c ^ pw_f(r)) << 4); }
__device__ __forceinline__ int pw_bpos(int n, int c) { return c ^ ((n >> 1) & 7); }
__device__ __forceinline__ int pw_mpos(int r, int p) { return p ^ ((r >> 3) & 1); }

template <bool CACHED>
__global__ __launch_bounds__(256) void spmm_panels_w4_kernel(const uint8_t* __restrict__ vp,
                                                             const uint8_t* __restrict__ mp, int64_t R, int64_t Kd,
                                                             const uint16_t* __restrict__ Bt, int64_t ldbt, int64_t Nc,
                                                             float* __restrict__ C, int64_t ldc) {
  constexpr int BM = 256, BN = 256, FM = 4, FN = 4, NW = 4;
  constexpr int SA = BM * 64, SB = BN * 128, SM = BM * 32;   // values of a step, Bt of a step, metadata of 4
  constexpr int OFF_A = 0, OFF_B = 3 * SA, OFF_M = 3 * SA + 3 * SB;
  constexpr int A_INSTR = SA / 1024 / NW, B_INSTR = SB / 1024 / NW, M_INSTR = SM / 1024 / NW;
  static_assert(A_INSTR == 4 && B_INSTR == 8 && M_INSTR == 2, "loads per wave and stage");
  static_assert(OFF_M + 2 * SM == 160 * 1024, "LDS budget");
  extern __shared__ __align__(1024) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // XCD-aware tile order, row tiles grouped as in the eight-wave kernel
  const int ntm = (int)(R / BM), ntn = (int)((Nc + BN - 1) / BN);
  const int wg = xcd_remap(blockIdx.x, ntm * ntn);
  const int GM = Kd >= 4096 ? 8 : 4;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int KT = (int)(Kd / 64), KC = KT / 4;
  const uint32_t smem_base = lds_addr(smem);

  // Sources as 32-bit byte offsets from wave-uniform bases (the dispatch checks the 4 GiB bound).
  // values load t of a wave: LDS lines 8q .. 8q+7 of the stage (row pairs); lane -> line
  // 8q + lane/8, LDS chunk lane%8 = (row parity, position p) holding source chunk p ^ pw_f(row)
  uint32_t a_off[A_INSTR];
#pragma unroll
  for (int t = 0; t < A_INSTR; ++t) {
    const int q = 8 * (wave * A_INSTR + t) + (lane >> 3);
    const int cl = lane & 7, r = 2 * q + (cl >> 2), c = (cl & 3) ^ pw_f(r);
    a_off[t] = (uint32_t)(((m0 / 2 + q) * KT) * 128 + (r & 1) * 64 + c * 16);
  }
  // metadata load t: LDS rows 32q .. 32q+31 of 32 bytes; lane -> row 32q + lane/2, LDS half lane%2
  uint32_t m_off[M_INSTR];
#pragma unroll
  for (int t = 0; t < M_INSTR; ++t) {
    const int r = 32 * (wave * M_INSTR + t) + (lane >> 1);
    const int p = pw_mpos(r, lane & 1);
    const int64_t row = m0 + r;
    m_off[t] = (uint32_t)(((row >> 2) * KC) * 128 + (row & 3) * 32 + p * 16);
  }
  // Bt load t: LDS rows 8q .. 8q+7 of 128 bytes (columns of the tile); columns past Nc read the last
  uint32_t b_off[B_INSTR];
#pragma unroll
  for (int t = 0; t < B_INSTR; ++t) {
    const int n = 8 * (wave * B_INSTR + t) + (lane >> 3);
    int64_t col = n0 + n;
    col = col < Nc ? col : Nc - 1;
    b_off[t] = (uint32_t)(2 * (col * ldbt + 8 * pw_bpos(n, lane & 7)));
  }
  // Batch s (stage s of the ring, slot s % 3): part 1 = the 8 Bt loads, part 2 = the 4 values
  // loads and, when s % 4 == 0, the 2 loads of metadata chunk s / 4 (slot (s / 4) % 2).  Stages
  // past the end repeat the last one into slots that are never read again.
  auto dma_b = [&](int s, int t) {
    const int sc = s < KT ? s : KT - 1;
    dma16s(b_off[t], Bt + (int64_t)sc * 64, uniform(smem_base + OFF_B + (s % 3) * SB + (wave * B_INSTR + t) * 1024));
  };
  auto dma_a = [&](int s, int t) {
    const int sc = s < KT ? s : KT - 1;
    dma16s(a_off[t], vp + (int64_t)sc * 128, uniform(smem_base + OFF_A + (s % 3) * SA + (wave * A_INSTR + t) * 1024));
  };
  auto dma_m = [&](int s, int t) {
    const int c = (s >> 2) < KC ? (s >> 2) : KC - 1;
    dma16s(m_off[t], mp + (int64_t)c * 128,
           uniform(smem_base + OFF_M + ((s >> 2) & 1) * SM + (wave * M_INSTR + t) * 1024));
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // v_smfmac_f32_32x32x32_bf16: lane l holds A row l%32 with the 8 kept values of dense k
  // 16*(l/32)..+15 of the instruction's 32 (index operand: the nibbles of those 4 groups); B
  // column l%32 with k = 8*(l/32)..+7 in elements 0..7 and k = 16 + 8*(l/32)..+7 in 8..15.
  const int l32 = lane & 31, aa = lane >> 5;
  // operand q of half h of stage s: q < 4 values fragment q; 4 <= q < 12 Bt fragment (q-4)/2, part (q-4)%2
  auto read_op = [&](int s, int h, int q, bf16x8 (&a)[FM], bf16x16 (&b)[FN]) {
    if (q < 4) {
      const int r = (wm * FM + q) * 32 + l32;
      a[q] = *reinterpret_cast<const bf16x8*>(smem + OFF_A + (s % 3) * SA + pw_apos(r, 2 * h + aa));
    } else {
      const int j = (q - 4) >> 1, part = (q - 4) & 1;
      const int n = wn * 128 + 32 * j + l32;
      const unsigned char* row = smem + OFF_B + (s % 3) * SB + n * 128;
      reinterpret_cast<bf16x8*>(&b[j])[part] =
          *reinterpret_cast<const bf16x8*>(row + (pw_bpos(n, 4 * h + 2 * part + aa) << 4));
    }
  };
  auto read_m = [&](int s, int i, u32x2 (&mm)[FM]) {
    const int r = (wm * FM + i) * 32 + l32, u = s & 3;
    mm[i] = *reinterpret_cast<const u32x2*>(smem + OFF_M + ((s >> 2) & 1) * SM + r * 32 + (pw_mpos(r, u >> 1) << 4) +
                                            8 * (u & 1));
  };
  // The 16 matrix instructions of half h; after matrix instruction m, mem(m).  Scheduling
  // barriers keep that order, so each memory instruction issues while a matrix instruction runs.
  auto half = [&](int h, const bf16x8 (&a)[FM], const bf16x16 (&b)[FN], const u32x2 (&mm)[FM], auto mem) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int j = m >> 2, i = m & 3;
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[i], b[j], acc[i][j], (int)(mm[i][h] >> (16 * aa)), 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mem(m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Step kt (its first-half operands in a0, b0 and its metadata in mmc, read during step kt-1):
  //   half 0: read stage kt's second-half operands into a1, b1; issue part 2 of batch kt+2 (slot
  //           (kt+2)%3 held stage kt-1, read completely before the previous barrier);
  //   wait for batch kt+1 (batch kt+2, 12 loads or 14 with a metadata chunk, may stay in
  //   flight); barrier: stage kt+1 is in LDS for every wave, every wave has read all of stage kt;
  //   half 1: read stage kt+1's first-half operands into a0, b0 and its metadata into mmn; issue
  //           part 1 of batch kt+3 into slot kt%3.
  bf16x8 a0[FM], a1[FM];
  bf16x16 b0[FN], b1[FN];
  u32x2 mmA[FM], mmB[FM];
  auto step = [&](int kt, u32x2 (&mmc)[FM], u32x2 (&mmn)[FM], auto waitf) {
    const int s2 = kt + 2, s3 = kt + 3;
    const bool meta2 = (s2 & 3) == 0;
    half(0, a0, b0, mmc, [&](int m) {
      if (m < 12) read_op(kt, 1, m, a1, b1);
      if ((m & 3) == 1) dma_a(s2, m >> 2);
      if (meta2 && (m == 3 || m == 11)) dma_m(s2, m >> 3);
    });
    waitf();
    lds_barrier();
    half(1, a1, b1, mmc, [&](int m) {
      if (m < 12) read_op(kt + 1, 0, m, a0, b0);
      else read_m(kt + 1, m - 12, mmn);
      if ((m & 1) == 0) dma_b(s3, m >> 1);
    });
  };
  // prologue: batches 0 and 1 whole and part 1 of batch 2; batch 0 has landed when at most the
  // 20 loads issued after it are in flight
#pragma unroll
  for (int t = 0; t < B_INSTR; ++t) dma_b(0, t);
#pragma unroll
  for (int t = 0; t < A_INSTR; ++t) dma_a(0, t);
#pragma unroll
  for (int t = 0; t < M_INSTR; ++t) dma_m(0, t);
#pragma unroll
  for (int t = 0; t < B_INSTR; ++t) dma_b(1, t);
#pragma unroll
  for (int t = 0; t < A_INSTR; ++t) dma_a(1, t);
#pragma unroll
  for (int t = 0; t < B_INSTR; ++t) dma_b(2, t);
  wait_vmcnt<20>();
  lds_barrier();
#pragma unroll
  for (int q = 0; q < 12; ++q) read_op(0, 0, q, a0, b0);
#pragma unroll
  for (int i = 0; i < FM; ++i) read_m(0, i, mmA);
  // KT is a multiple of 4; batch kt+2 carries a metadata chunk when kt % 4 == 2
  for (int kt = 0; kt < KT; kt += 4) {
    step(kt, mmA, mmB, [] { wait_vmcnt<12>(); });
    step(kt + 1, mmB, mmA, [] { wait_vmcnt<12>(); });
    step(kt + 2, mmA, mmB, [] { wait_vmcnt<14>(); });
    step(kt + 3, mmB, mmA, [] { wait_vmcnt<12>(); });
  }
  wait_vmcnt<0>();   // drain: no load may land in LDS after the workgroup ends

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * 128 + 32 * j + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * aa + (e & 3);
        if (col < Nc) {
          if constexpr (CACHED) C[row * ldc + col] = acc[i][j][e];
          else __builtin_nontemporal_store(acc[i][j][e], C + row * ldc + col);
        }
      }
    }
  }
}

// Conditions: bf16 (checked by the caller), whole 256-row tiles and 256-column chunks, 16-byte
// aligned operands and Bt rows, every operand addressable with 32-bit byte offsets.
bool spmm_panels_ok(const void* values, const uint8_t* meta, const void* Bt, int64_t ldbt, int64_t R, int64_t K,
                    int64_t Nc) {
  return R % 256 == 0 && K % 256 == 0 && ldbt % 8 == 0 && (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 16 == 0 &&
         (uintptr_t)Bt % 16 == 0 && R * K < (int64_t(1) << 32) && Nc * ldbt * 2 < (int64_t(1) << 32);
}

hipError_t launch_spmm_nm_t_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                   int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  if (!spmm_panels_ok(values, meta, Bt, ldbt, R, K, Nc)) return hipErrorNotSupported;
  constexpr int LDS = 160 * 1024;
  const bool cached = R * Nc * 4 <= kW4CachedCBytes;
  auto kern = cached ? spmm_panels_w4_kernel<true> : spmm_panels_w4_kernel<false>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  const int64_t ntiles = (R / 256) * ((Nc + 255) / 256);
  if (ntiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(256), (size_t)LDS, s, (const uint8_t*)values, meta, R, K,
                     (const uint16_t*)Bt, ldbt, Nc, C, ldc);
  return hipGetLastError();
}

}  // namespace nms
