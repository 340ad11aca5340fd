// 2:4 SpMM with the dense operand given K-contiguous ("NT" form), gfx950.
//
// Product: C[r][n] = sum_k A[r][k] Bt[n][k], A in 2:4 form (values + nibbles)
// ("Success story: ESPLAG", Research Topic: the SpMM of a 2:4 layer; "To 2:4
// Sparsity and Beyond", abstract: 2:4 weights in every FFN matmul).  Bt is the
// dense operand with its reduction index contiguous -- the token-major layout
// in which an FFN's activations [tokens][d_model] are usually kept -- which is
// also the order v_smfmac wants for its B operand (each lane holds 16 k values
// of one column).  Both operands therefore go from HBM to LDS with
// direct-to-LDS loads, as whole rows, and nothing is transposed on the way: the
// kernel's instruction stream is operand reads from LDS and matrix
// instructions.  A transpose pass (nm_transpose_bf16_kernel below) turns a
// row-major B [K][Nc] into Bt once; every row tile of the SpMM then reads Bt's
// panels directly.
//
// v_smfmac_f32_32x32x32_bf16 on gfx950: lane l holds A row l%32 with the 8 kept
// values of dense k 16*(l/32)..+15 (index operand: one nibble p0 | p1 << 2 per
// group of 4, group 0 in bits 0..3 -- the stored metadata order); B column l%32
// with k = 8*(l/32)..+7 in elements 0..7 and k = 16 + 8*(l/32)..+7 in elements
// 8..15; C column l%32, element e at row 8*(e/4) + 4*(l/32) + e%4.
//
// Loads (measured on gfx950): the vector L1 of a CU spends about two cycles per
// 128-byte line an instruction touches, however few of its bytes are used, so
// every operand is fetched as whole lines: values two 64-k steps at a time (128
// bytes of a row), metadata four steps at a time (32 bytes of a row), Bt one
// step at a time (128 bytes of a column), each into two LDS buffers (144 KB).
// The 16-byte chunks of a 128-byte LDS row are XOR-swizzled by (row >> 1) & 7
// and the two 16-byte halves of a 32-byte metadata row swap every 8 rows, so
// the operand reads of 16 (32) consecutive rows are free of bank conflicts.
// 8 waves (two per SIMD) own 128 x 64 of the 256 x 256 tile each, 4 x 2
// fragments with accumulators in VGPRs.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "prep_bodies.hpp"

namespace nms {

__device__ __forceinline__ int nt_apos(int r, int c) { return c ^ ((r >> 1) & 7); }

// largest C (bytes) written with ordinary stores
constexpr int64_t kCachedCBytes = int64_t(160) << 20;
__device__ __forceinline__ int nt_bpos(int n, int c) { return c ^ ((n >> 1) & 7); }
__device__ __forceinline__ int nt_mpos(int r, int p) { return p ^ ((r >> 3) & 1); }

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct NtCfg {
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int SA = BM * 128;     // values of two steps
  static constexpr int SM = BM * 32;      // metadata of four steps
  static constexpr int SB = BN * 128;     // Bt of one step
  static constexpr int OFF_A = 0, OFF_B = 2 * SA, OFF_M = 2 * SA + 2 * SB;
  static constexpr int LDS = 2 * (SA + SB + SM);
  static constexpr int A_INSTR = SA / 1024 / NW, M_INSTR = SM / 1024 / NW, B_INSTR = SB / 1024 / NW;
  static_assert(A_INSTR >= 1 && M_INSTR >= 1 && B_INSTR >= 1, "every wave loads a share of each operand");
  static_assert(SA % (1024 * NW) == 0 && SM % (1024 * NW) == 0 && SB % (1024 * NW) == 0, "tiling");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "fragments");
  static_assert(A_INSTR + M_INSTR + B_INSTR <= 63, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// OutT: float (fp32 C) or uint16_t (bf16 C, each fp32 sum rounded to nearest even).
// LR: add a low-rank adapter term U Tt^T to the accumulators before they are stored (U [R][ldu]
// bf16, Tt [Nc][rank] fp32, rank a multiple of 16; unused otherwise).
// VNM (= M, 0 for off): instead of storing C, prune h = ReLU(bf16(C))^T (columns of C are
// tokens) to V:N:M with V = vnm_v tokens (64, 128 or 256) and M rows of C (4, 8 or 16), writing
// h's values, nibbles and column choices (hv, hm, hc in the layout of prune_act_venom; R and Nc
// multiples of 256).
template <int BM, int BN, int WAVES_M, int WAVES_N, typename OutT, bool LR, int VNM = 0, bool CACHED = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void spmm_nt_kernel(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, int64_t R, int64_t Kd,
    const uint16_t* __restrict__ Bt, int64_t ldbt, int64_t Nc, OutT* __restrict__ C, int64_t ldc,
    const uint16_t* __restrict__ U, int64_t ldu, const float* __restrict__ Tt, int rank,
    uint16_t* __restrict__ hv, uint8_t* __restrict__ hm, uint8_t* __restrict__ hc, int vnm_v) {
  using Cfg = NtCfg<BM, BN, WAVES_M, WAVES_N>;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  extern __shared__ __align__(1024) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int ntm = (int)((R + BM - 1) / BM), ntn = (int)((Nc + BN - 1) / BN);
  const int nwg = ntm * ntn;
  const int wg = xcd_remap(blockIdx.x, nwg);
  // row tiles per group of the tile order: with long rows (K >= 4096: 64 or more steps per tile,
  // the training step's products) eight row tiles share each column panel while they run, at
  // K = 2048 four (measured: 591 -> 575 us at 4096 x 16384 x 8192, 586 -> 583 at 16384 x 4096 x
  // 8192; 86 -> 97 us at 8192 x 2048 x 4096 with eight)
  const int GM = Kd >= 4096 ? 8 : 4;
  const int grp = wg / (GM * ntn);
  const int first_m = grp * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int within = wg - grp * GM * ntn;
  const int tm = first_m + within % gsz, tn = within / gsz;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int64_t vrow = Kd / 2, mrow = Kd / 8;
  const int KT = (int)(Kd / 64);            // a multiple of 4
  const int jlast = KT / 2 - 1, clast = KT / 4 - 1;
  const uint32_t smem_base = lds_addr(smem);

  // Sources as 32-bit byte offsets from wave-uniform bases (the dispatch guarantees every operand
  // is smaller than 4 GiB).
  // values, instruction t: LDS rows 8q .. 8q+7 of 128 bytes; lane -> row 8q + lane/8, chunk lane%8
  uint32_t a_off[Cfg::A_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::A_INSTR; ++t) {
    const int r = 8 * (wave * Cfg::A_INSTR + t) + (lane >> 3);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    a_off[t] = (uint32_t)(2 * (row * vrow + 8 * nt_apos(r, lane & 7)));
  }
  // metadata, instruction t: LDS rows 32q .. 32q+31 of 32 bytes; lane -> row 32q + lane/2, piece lane%2
  uint32_t m_off[Cfg::M_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::M_INSTR; ++t) {
    const int r = 32 * (wave * Cfg::M_INSTR + t) + (lane >> 1);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    m_off[t] = (uint32_t)(row * mrow + 16 * nt_mpos(r, lane & 1));
  }
  // Bt, instruction t: LDS rows 8q .. 8q+7 of 128 bytes; lane -> row 8q + lane/8, chunk lane%8
  uint32_t b_off[Cfg::B_INSTR];
#pragma unroll
  for (int t = 0; t < Cfg::B_INSTR; ++t) {
    const int n = 8 * (wave * Cfg::B_INSTR + t) + (lane >> 3);
    int64_t col = n0 + n;
    col = col < Nc ? col : Nc - 1;
    b_off[t] = (uint32_t)(2 * (col * ldbt + 8 * nt_bpos(n, lane & 7)));
  }
  auto issue_a = [&](int buf, int j) {   // values of steps 2j, 2j+1
    const uint32_t st = smem_base + Cfg::OFF_A + buf * Cfg::SA;
    const uint16_t* base = values + (int64_t)j * 64;
#pragma unroll
    for (int t = 0; t < Cfg::A_INSTR; ++t) dma16s(a_off[t], base, uniform(st + (wave * Cfg::A_INSTR + t) * 1024));
  };
  auto issue_m = [&](int buf, int c) {   // metadata of steps 4c .. 4c+3
    const uint32_t st = smem_base + Cfg::OFF_M + buf * Cfg::SM;
    const uint8_t* base = meta + (int64_t)c * 32;
#pragma unroll
    for (int t = 0; t < Cfg::M_INSTR; ++t) dma16s(m_off[t], base, uniform(st + (wave * Cfg::M_INSTR + t) * 1024));
  };
  auto issue_b = [&](int buf, int kt) {
    const uint32_t st = smem_base + Cfg::OFF_B + buf * Cfg::SB;
    const uint16_t* base = Bt + (int64_t)kt * 64;
#pragma unroll
    for (int t = 0; t < Cfg::B_INSTR; ++t) dma16s(b_off[t], base, uniform(st + (wave * Cfg::B_INSTR + t) * 1024));
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int l32 = lane & 31, aa = lane >> 5;
  auto step = [&](int kt, auto issue_b_next, auto issue_am_next) {
    const int s = kt & 1, u = kt & 3;
    const unsigned char* As = smem + Cfg::OFF_A + ((kt >> 1) & 1) * Cfg::SA;
    const unsigned char* Ms = smem + Cfg::OFF_M + ((kt >> 2) & 1) * Cfg::SM;
    const unsigned char* Bs = smem + Cfg::OFF_B + (kt & 1) * Cfg::SB;
    u32x2 mm[FM];
    bf16x8 a[2][FM];
    bf16x16 b[2][FN];
    auto operands = [&](int h) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = (wm * FM + i) * 32 + l32;
        a[h][i] = *reinterpret_cast<const bf16x8*>(As + r * 128 + (nt_apos(r, 4 * s + 2 * h + aa) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * Cfg::WN + 32 * j + l32;
        const unsigned char* row = Bs + n * 128;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(row + (nt_bpos(n, 4 * h + aa) << 4));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(row + (nt_bpos(n, 4 * h + 2 + aa) << 4));
        b[h][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
    };
    auto mfma = [&](int h) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[h][i], b[h][j], acc[i][j],
                                                               (int)(mm[i][h] >> (16 * aa)), 0, 0);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = (wm * FM + i) * 32 + l32;
      mm[i] = *reinterpret_cast<const u32x2*>(Ms + r * 32 + (nt_mpos(r, u >> 1) << 4) + 8 * (u & 1));
    }
    // Bt of the next step is issued first (one step of lookahead); the values and metadata stages
    // (two and four steps ahead) only once the first half's matrix instructions are issued, so
    // that they do not delay the Bt loads
    issue_b_next();
    operands(0);
    __builtin_amdgcn_sched_barrier(0);
    operands(1);
    mfma(0);
    __builtin_amdgcn_sched_barrier(0);
    issue_am_next();
    mfma(1);
  };

  // Step kt needs values super-stage kt/2 (loaded during step kt-2), metadata chunk kt/4 (during
  // step kt-4) and Bt step kt (during step kt-1, as the first loads of that step).  The wait before
  // step kt lets through the loads issued after Bt step kt: a values super-stage when kt-1 is even,
  // a metadata chunk when kt-1 is a multiple of 4.  Past the end the loads repeat the last stage
  // into buffers that are never read again, so every step looks alike.
  issue_a(0, 0);
  issue_m(0, 0);
  issue_b(0, 0);
  // Low-rank adapter operands (LR): U in 64-column stages through the values buffers, Tt in
  // 32-column fp32 stages through the Bt buffers, rows of 128 bytes with the same swizzles.  Chunks
  // past the adapter's width repeat its last chunk (never read as operands).
  auto issue_u = [&](int buf, int u) {
    const uint32_t st = smem_base + Cfg::OFF_A + buf * Cfg::SA;
    const int nch = (rank - 64 * u) / 8 < 8 ? (rank - 64 * u) / 8 : 8;
#pragma unroll
    for (int t = 0; t < Cfg::A_INSTR; ++t) {
      const int r = 8 * (wave * Cfg::A_INSTR + t) + (lane >> 3);
      int64_t row = m0 + r;
      row = row < R ? row : R - 1;
      int c = nt_apos(r, lane & 7);
      c = c < nch ? c : nch - 1;
      dma16s((uint32_t)(2 * (row * ldu + 64 * u + 8 * c)), U, uniform(st + (wave * Cfg::A_INSTR + t) * 1024));
    }
  };
  auto issue_tt = [&](int buf, int s) {
    const uint32_t st = smem_base + Cfg::OFF_B + buf * Cfg::SB;
    const int nch = (rank - 32 * s) / 4 < 8 ? (rank - 32 * s) / 4 : 8;
#pragma unroll
    for (int t = 0; t < Cfg::B_INSTR; ++t) {
      const int n = 8 * (wave * Cfg::B_INSTR + t) + (lane >> 3);
      int64_t col = n0 + n;
      col = col < Nc ? col : Nc - 1;
      int c = nt_bpos(n, lane & 7);
      c = c < nch ? c : nch - 1;
      dma16s((uint32_t)(4 * (col * rank + 32 * s + 4 * c)), Tt, uniform(st + (wave * Cfg::B_INSTR + t) * 1024));
    }
  };
  auto body = [&](int kt, auto wait) {
    wait();
    lds_barrier();   // step kt's operands are in LDS for every wave; every wave is done with step kt-1
    auto am = [&] {
      if constexpr (LR) {
        // the first adapter stage of U takes the place of the repeated last values super-stage
        if ((kt & 1) == 0 && (kt >> 1) + 1 > jlast) issue_u(((kt >> 1) + 1) & 1, 0);
        else if ((kt & 1) == 0) issue_a(((kt >> 1) + 1) & 1, (kt >> 1) + 1);
      } else {
        if ((kt & 1) == 0) issue_a(((kt >> 1) + 1) & 1, (kt >> 1) + 1 <= jlast ? (kt >> 1) + 1 : jlast);
      }
      if ((kt & 3) == 0) issue_m(((kt >> 2) + 1) & 1, (kt >> 2) + 1 <= clast ? (kt >> 2) + 1 : clast);
    };
    step(kt, [&] {
      if constexpr (LR) {
        if (kt + 1 == KT) {   // the first Tt stage takes the place of the repeated last Bt step
          issue_tt(KT & 1, 0);
          return;
        }
      }
      issue_b((kt + 1) & 1, kt + 1 < KT ? kt + 1 : KT - 1);
    }, am);
  };
  for (int kt = 0; kt < KT; kt += 4) {
    body(kt, [] { wait_vmcnt<0>(); });
    body(kt + 1, [] { wait_vmcnt<Cfg::A_INSTR + Cfg::M_INSTR>(); });
    body(kt + 2, [] { wait_vmcnt<0>(); });
    body(kt + 3, [] { wait_vmcnt<Cfg::A_INSTR>(); });
  }
  wait_vmcnt<0>();   // drain: no load may land in LDS after the workgroup ends

  if constexpr (LR) {
    // Adapter steps s = 0 .. ceil(rank/32)-1 after the sparse ones: acc[i][j] += U[rows of
    // fragment i][32s..32s+31] . Tt[columns of fragment j][32s..32s+31], one 16-wide slice at a
    // time by v_mfma_f32_32x32x16_bf16 (A operand: U row l%32, k = 8*(l/32)..+7; B operand: Tt row
    // l%32, the same k; the result layout is the accumulators' own).  Tt stage s sits in Bt buffer
    // (KT + s) % 2 and U stage s/2 in values buffer (jlast + 1 + s/2) % 2; each step issues the
    // next stages after its barrier, as the sparse steps do.  Tt is fp32: each value enters as two
    // bf16 parts (its top 16 bits, then the remainder rounded to nearest even), about 16
    // significant bits in all.  Rows and columns past the matrix read the last one; their sums are
    // never stored.
    const int S = (rank + 31) / 32, NU = (rank + 63) / 64;
    for (int s = 0; s < S; ++s) {
      wait_vmcnt<0>();
      lds_barrier();
      if (s + 1 < S) issue_tt((KT + s + 1) & 1, s + 1);
      if ((s & 1) == 0 && (s >> 1) + 1 < NU) issue_u((jlast + 2 + (s >> 1)) & 1, (s >> 1) + 1);
      const unsigned char* Us = smem + Cfg::OFF_A + ((jlast + 1 + (s >> 1)) & 1) * Cfg::SA;
      const unsigned char* Ts = smem + Cfg::OFF_B + ((KT + s) & 1) * Cfg::SB;
      const int nh = rank - 32 * s >= 32 ? 2 : 1;
      for (int h = 0; h < nh; ++h) {
        const int hu = 2 * (s & 1) + h;   // 16-wide slice within the U stage
        bf16x8 ua[FM], th[FN], tl[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = (wm * FM + i) * 32 + l32;
          ua[i] = *reinterpret_cast<const bf16x8*>(Us + r * 128 + (nt_apos(r, 2 * hu + aa) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = wn * Cfg::WN + 32 * j + l32;
          const unsigned char* row = Ts + n * 128;
          split_bf16x8(*reinterpret_cast<const f32x4*>(row + (nt_bpos(n, 4 * h + 2 * aa) << 4)),
                       *reinterpret_cast<const f32x4*>(row + (nt_bpos(n, 4 * h + 2 * aa + 1) << 4)), th[j], tl[j]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[i], th[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[i], tl[j], acc[i][j], 0, 0, 0);
          }
      }
    }
    wait_vmcnt<0>();
  }

  if constexpr (VNM > 0) {
    static_assert(BM == 256 && BN == 256 && !LR, "the V:N:M epilogue takes whole 256 x 256 tiles");
    static_assert(VNM == 4 || VNM == 8 || VNM == 16, "M");
    constexpr int M = VNM, NG = 256 / M;   // groups of the tile's 256 rows
    const int V = vnm_v, NB = 256 / V;     // V-blocks of the tile's 256 tokens
    // 1. h = ReLU(bf16(acc)) into LDS, token-major: ht[n][r] for the tile's 256 tokens n and 256
    //    rows r of C, 260 elements per token (each lane's 8-byte writes of 32 tokens then fall on
    //    distinct banks)
    constexpr int HP = 260;
    uint16_t* ht = reinterpret_cast<uint16_t*>(smem);
    double* l1 = reinterpret_cast<double*>(smem + 256 * HP * 2);   // [NB][256]
    uint32_t* cs = reinterpret_cast<uint32_t*>(l1 + 1024);          // [NB][NG]
    lds_barrier();   // every wave is done with the last step's operands
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * Cfg::WN + 32 * j + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * Cfg::WM + 32 * i + 8 * q + 4 * aa;
          uint32_t b[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint16_t x = f32_to_bf16_rne(acc[i][j][4 * q + u]);
            b[u] = Elem<uint16_t>::positive(x) ? x : 0u;
          }
          *reinterpret_cast<u32x2*>(ht + n * HP + r) = u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        }
      }
    __syncthreads();
    // 2. column norms: one lane per (V-block, row) adds h over the block's V tokens, in fp64 and
    //    token order (the sequence of additions of any sequential implementation)
    for (int u = tid; u < NB * 256; u += Cfg::NT) {
      const int vb = u >> 8, r = u & 255;
      double acc1 = 0.0;
      for (int n = 0; n < V; ++n) acc1 += (double)Elem<uint16_t>::to_f32(ht[(vb * V + n) * HP + r]);
      l1[u] = acc1;
    }
    __syncthreads();
    // 3. per (V-block, group of M rows): the 4 rows of largest norm, lower row on ties
    const int64_t Gh = R / M;   // groups per token of h
    for (int u = tid; u < NB * NG; u += Cfg::NT) {
      const int vb = u / NG, g = u % NG;
      double k[M];
#pragma unroll
      for (int p = 0; p < M; ++p) k[p] = l1[vb * 256 + M * g + p];
      uint32_t packed = 0;
      int c = 0;
#pragma unroll
      for (int p = 0; p < M; ++p)
        if (rank_f64<M>(k, p) < 4) {
          packed |= (uint32_t)p << (8 * c);
          ++c;
        }
      cs[u] = packed;
      *reinterpret_cast<uint32_t*>(hc + ((n0 / V + vb) * Gh + m0 / M + g) * 4) = packed;
    }
    __syncthreads();
    // 4. per (token, 8 groups): 2 of the group's 4 chosen rows by magnitude (lower on ties);
    //    32 bytes of values and 4 bytes of nibbles per token and octet of groups
    constexpr int NO = NG / 8;   // octets of groups per token
    for (int it = tid; it < 256 * NO; it += Cfg::NT) {
      const int n = it / NO, g0 = (it % NO) * 8, vb = n / V;
      const uint16_t* trow = ht + n * HP;
      uint32_t out[8];
      uint32_t nibs = 0;
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint32_t packed = cs[vb * NG + g0 + gi];
        uint32_t x[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[jj] = trow[M * (g0 + gi) + ((packed >> (8 * jj)) & 0xFF)];
        const uint32_t nib = select24_bf16(x[0], x[1], x[2], x[3]);
        const uint32_t d01 = x[0] | (x[1] << 16), d23 = x[2] | (x[3] << 16);
        const uint32_t j0 = nib & 3, j1 = nib >> 2;
        out[gi] = __builtin_amdgcn_perm(d23, d01, (j0 * 0x202u + 0x100u) | ((j1 * 0x202u + 0x100u) << 16));
        nibs |= nib << (4 * gi);
      }
      const int64_t tok = n0 + n, grp = m0 / M + g0;
      u32x4* dv = reinterpret_cast<u32x4*>(hv + tok * (Gh * 2) + grp * 2);
      dv[0] = u32x4{out[0], out[1], out[2], out[3]};
      dv[1] = u32x4{out[4], out[5], out[6], out[7]};
      *reinterpret_cast<uint32_t*>(hm + tok * (Gh / 2) + grp / 2) = nibs;
    }
    return;
  }

  // CACHED: C leaves with ordinary stores (chosen while C fits the last-level cache comfortably:
  // each round's burst of tiles is then absorbed there); otherwise with non-temporal ones, which
  // keep C from evicting the operands the later tiles still read
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * Cfg::WN + 32 * j + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * Cfg::WM + 32 * i + 8 * (e >> 2) + 4 * aa + (e & 3);
        if (row < R && col < Nc) {
          OutT v;
          if constexpr (sizeof(OutT) == 4) v = acc[i][j][e];
          else v = f32_to_bf16_rne(acc[i][j][e]);
          if constexpr (CACHED) C[row * ldc + col] = v;
          else __builtin_nontemporal_store(v, C + row * ldc + col);
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, typename OutT, bool LR = false, int VNM = 0, bool CACHED = false>
static hipError_t run_nt(const void* values, const uint8_t* meta, int64_t R, int64_t Kd, const void* Bt, int64_t ldbt,
                         int64_t Nc, OutT* C, int64_t ldc, hipStream_t s, const void* U = nullptr, int64_t ldu = 0,
                         const float* Tt = nullptr, int rank = 0, uint16_t* hv = nullptr, uint8_t* hm = nullptr,
                         uint8_t* hc = nullptr, int vnm_v = 0) {
  using Cfg = NtCfg<BM, BN, WAVES_M, WAVES_N>;
  auto kern = spmm_nt_kernel<BM, BN, WAVES_M, WAVES_N, OutT, LR, VNM, CACHED>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  const int64_t ntiles = ((R + BM - 1) / BM) * ((Nc + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg::NT), (size_t)Cfg::LDS, s, (const uint16_t*)values, meta,
                     R, Kd, (const uint16_t*)Bt, ldbt, Nc, C, ldc, (const uint16_t*)U, ldu, Tt, rank, hv, hm, hc, vnm_v);
  return hipGetLastError();
}

// Conditions: bf16, whole 256-k chunks (four steps), 16-byte loads of values, metadata and Bt
// rows, and every operand addressable with 32-bit byte offsets.
bool spmm_nt_ok(const void* values, const uint8_t* meta, const void* Bt, int64_t ldbt, int64_t R, int64_t Nc,
                int64_t Kd) {
  return Kd % 256 == 0 && ldbt % 8 == 0 && (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 16 == 0 &&
         (uintptr_t)Bt % 16 == 0 && R * Kd < (int64_t(1) << 32) && Nc * ldbt * 2 < (int64_t(1) << 32);
}

hipError_t launch_spmm_nm_nt_dma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                 int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s) {
  if (R * Nc * 4 <= kCachedCBytes)
    return run_nt<256, 256, 2, 4, float, false, 0, true>(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
  return run_nt<256, 256, 2, 4>(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
}

hipError_t launch_spmm_nm_nt_dma_bf16out(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                         int64_t ldbt, int64_t Nc, uint16_t* C, int64_t ldc, hipStream_t s) {
  return run_nt<256, 256, 2, 4>(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
}

hipError_t launch_spmm_nm_t_relu_venom(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                      int64_t ldbt, int64_t Nc, int V, int M, void* hv, uint8_t* hm, uint8_t* hc,
                                      hipStream_t s) {
  // the fused epilogue's conditions: V in {64, 128, 256} and M in {4, 8, 16} with whole 256 x 256
  // tiles, the pipelined SpMM's own conditions, 16-byte value rows and 4-byte metadata and
  // column-choice words
  if ((V != 64 && V != 128 && V != 256) || (M != 4 && M != 8 && M != 16) || R % 256 != 0 || Nc % 256 != 0 ||
      !spmm_nt_ok(values, meta, Bt, ldbt, R, Nc, K) || (uintptr_t)hv % 16 != 0 || (uintptr_t)hm % 4 != 0 ||
      (uintptr_t)hc % 4 != 0)
    return hipErrorNotSupported;
  auto go = [&](auto MM) {
    return run_nt<256, 256, 2, 4, float, false, decltype(MM)::value>(values, meta, R, K, Bt, ldbt, Nc, (float*)nullptr,
                                                                     0, s, nullptr, 0, nullptr, 0, (uint16_t*)hv, hm,
                                                                     hc, V);
  };
  return M == 4 ? go(std::integral_constant<int, 4>{}) : M == 8 ? go(std::integral_constant<int, 8>{})
                                                                : go(std::integral_constant<int, 16>{});
}

hipError_t launch_spmm_nm_nt_dma_lowrank(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                         int64_t ldbt, int64_t Nc, const void* U, int64_t ldu, const float* Tt,
                                         int rank, float* C, int64_t ldc, hipStream_t s) {
  if (R * Nc * 4 <= kCachedCBytes)
    return run_nt<256, 256, 2, 4, float, true, 0, true>(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s, U, ldu, Tt,
                                                        rank);
  return run_nt<256, 256, 2, 4, float, true>(values, meta, R, K, Bt, ldbt, Nc, C, ldc, s, U, ldu, Tt, rank);
}

// ---------------------------------------------------------------------------
// Transpose of a bf16 matrix (prep_bodies.hpp): 64 x 64 tiles, one per wave.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nm_transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                int64_t R, int64_t Cn, uint16_t* __restrict__ dst,
                                                                int64_t ldd) {
  transpose_bf16_body(blockIdx.x, src, lds, R, Cn, dst, ldd);
}

hipError_t launch_nm_transpose(int dt, const void* src, int64_t lds, int64_t R, int64_t Cn, void* dst, int64_t ldd,
                               hipStream_t s) {
  if (dt != DT_BF16) return hipErrorNotSupported;
  const int64_t tiles = ((R + 63) / 64) * ((Cn + 63) / 64);
  hipLaunchKernelGGL(nm_transpose_bf16_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s,
                     (const uint16_t*)src, lds, R, Cn, (uint16_t*)dst, ldd);
  return hipGetLastError();
}

}  // namespace nms
