// V:N:M SpMM with the gathered dense rows loaded straight into registers (gfx950).
//
// Product ("To 2:4 Sparsity and Beyond", abstract; "Success story: ESPLAG", Solution):
//   C[r][n] = sum_g sum_s vals[r][2g+s] * B[g*M + colsel[r/V][g][p_s(r,g)]][n]
// i.e. 2:4 over the four columns each V-row block keeps per group of M, with the
// kept rows of B gathered through colsel.  Every V-row block gathers a different
// half (M = 8) of B's rows, so a tile can share a gathered B element only among
// the rows of its own block: a 64-row block uses each element 64 times.  Staging
// such an operand through LDS (written once, read back once per use) costs as
// much LDS traffic as the matrix instructions can absorb; this kernel never
// stages B.  Each wave loads the B values its own matrix instructions need,
// directly in the order the instruction takes them:
//
//  * v_smfmac_f32_32x32x32_bf16 takes B column l%32 in lane l, with dense k
//    8*(l/32)..+7 in elements 0..7 and 16 + 8*(l/32)..+7 in elements 8..15.  A
//    wave owns 64 columns as two fragments, f = 0 on the even and f = 1 on the
//    odd columns: lane l then needs columns 2c and 2c+1 (c = l%32) -- one
//    aligned dword of a B row -- of 16 rows per 32-k half.  One
//    buffer_load_dword per row slot gives lanes 0-31 one gathered row and lanes
//    32-63 another (two 128-byte lines, the whole line used), so 16 loads fill a
//    half; v_perm pairs the bf16 halves of two rows into the fragments' operand
//    dwords.  The per-lane row offsets come from a table of gathered-row byte
//    offsets that each workgroup builds in LDS from colsel once, read back as
//    broadcast 16-byte LDS reads (four per half).
//  * The sparse operand (values + 2:4 metadata over the gathered columns) is
//    shared by the four waves of a workgroup and staged in LDS by direct
//    global->LDS loads of whole 128-byte rows, two 64-k steps at a time,
//    exactly as in the row-major SpMM.
//
// Tile: 64 rows (inside one V-row block; V % 64 == 0) x 256 columns, four waves
// of 64 x 64 (2 x 2 fragments, 64 accumulators), two workgroups per CU.  The B
// loads of step k+2 are issued during step k (three register sets of 32
// dwords); waits are explicit vmcnt counts of the fixed issue order, and each
// wait names the registers it publishes.  Tiles are dealt column-panel-major
// per XCD, so each XCD's L2 holds the B panels of its own tiles only.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {
namespace {

constexpr int VG_BM = 64;                       // rows per tile (inside one V-row block)
constexpr int VG_WAVES = 4;
constexpr int VG_NT = 64 * VG_WAVES;
constexpr int VG_BN = 64 * VG_WAVES;            // 64 columns per wave
constexpr int VG_AV = VG_BM * 128;              // values of a super-stage: 64 kept bf16 per row (two steps)
constexpr int VG_AM = VG_BM * 16;               // metadata of a super-stage: 16 bytes per row
constexpr int VG_ASTAGE = VG_AV + VG_AM;
constexpr int VG_AV_INSTR = VG_AV / 1024 / VG_WAVES;   // direct loads of values per wave and super-stage
constexpr int VG_AM_LANES = VG_BM / VG_WAVES;          // metadata rows per wave
constexpr int VG_LA = VG_AV_INSTR + 1;                 // vector-memory instructions of a super-stage per wave
constexpr int VG_LB = 32;                              // vector-memory instructions of a step's B rows per wave
constexpr int VG_TAB_STEP = 64 * 4;                    // table bytes per step: 64 gathered rows x u32 offset
static_assert(VG_AV_INSTR >= 1 && VG_AV % (1024 * VG_WAVES) == 0, "values loads per wave");
static_assert(VG_LA + VG_LB <= 63, "vmcnt range of the waits");

__device__ __forceinline__ int vg_apos(int r, int c) { return c ^ ((r >> 1) & 7); }

// One dword of B at byte offset voff of the wave's buffer; out of range reads give 0.
__device__ __forceinline__ uint32_t bload(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc) {
  uint32_t x;
  asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(x) : "v"(voff), "s"(rsrc));
  return x;
}

// Waits until at most N vector-memory instructions of this wave are outstanding; the 32
// registers named are those the wait publishes (the compiler may not touch them before it).
template <int N>
__device__ __forceinline__ void wait_set(uint32_t (&b)[32]) {
  asm volatile("s_waitcnt vmcnt(%32)"
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7]),
                 "+v"(b[8]), "+v"(b[9]), "+v"(b[10]), "+v"(b[11]), "+v"(b[12]), "+v"(b[13]), "+v"(b[14]),
                 "+v"(b[15]), "+v"(b[16]), "+v"(b[17]), "+v"(b[18]), "+v"(b[19]), "+v"(b[20]), "+v"(b[21]),
                 "+v"(b[22]), "+v"(b[23]), "+v"(b[24]), "+v"(b[25]), "+v"(b[26]), "+v"(b[27]), "+v"(b[28]),
                 "+v"(b[29]), "+v"(b[30]), "+v"(b[31])
               : "n"(N)
               : "memory");
}

}  // namespace

// Table position (in u32 entries within a step) of gathered row gk of the step: the loads of
// half h = gk / 32 read, for lanes of half hh = (gk / 8) % 2, slot e' = gk % 8 + 8 * ((gk / 16) % 2).
__device__ __forceinline__ int vg_tab_pos(int gk) {
  return ((gk >> 5) << 5) | (((gk >> 3) & 1) << 4) | (gk & 7) | (((gk >> 4) & 1) << 3);
}

__global__ __launch_bounds__(VG_NT, 2) void spmm_vnm_reg_kernel(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, const uint8_t* __restrict__ colsel,
    int64_t R, int64_t Kd, int V, int M, int64_t G, const uint16_t* __restrict__ B, int64_t ldb, int64_t Nc,
    float* __restrict__ C, int64_t ldc, int gm) {
  extern __shared__ __align__(1024) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int ntm = (int)((R + VG_BM - 1) / VG_BM), ntn = (int)((Nc + VG_BN - 1) / VG_BN);
  int tm, tn;
  panel_major_tile(blockIdx.x, ntm, ntn, gm, tm, tn);
  const int64_t m0 = (int64_t)tm * VG_BM, n0 = (int64_t)tn * VG_BN;
  const int64_t vblk = m0 / V;
  const int KT = (int)(Kd / 64);   // 64-k steps of the gathered dimension (even)
  const int64_t vrow = Kd / 2, mrow = Kd / 8;
  const uint32_t smem_base = lds_addr(smem);
  unsigned char* const a_lds = smem;
  uint32_t* const table = reinterpret_cast<uint32_t*>(smem + 2 * VG_ASTAGE);

  // ---- sparse operand: direct-to-LDS sources (as in the row-major SpMM) ----
  const uint16_t* a_src[VG_AV_INSTR];
#pragma unroll
  for (int t = 0; t < VG_AV_INSTR; ++t) {
    const int r = 8 * (wave * VG_AV_INSTR + t) + (lane >> 3);
    int64_t row = m0 + r;
    row = row < R ? row : R - 1;
    a_src[t] = values + row * vrow + 8 * vg_apos(r, lane & 7);
  }
  const uint8_t* m_src;
  {
    int64_t row = m0 + wave * VG_AM_LANES + (lane < VG_AM_LANES ? lane : 0);
    row = row < R ? row : R - 1;
    m_src = meta + row * mrow;
  }
  auto issue_a = [&](int j) {
    const uint32_t st = smem_base + (j & 1) * VG_ASTAGE;
#pragma unroll
    for (int t = 0; t < VG_AV_INSTR; ++t)
      dma16(a_src[t] + (int64_t)j * 64, uniform(st + (wave * VG_AV_INSTR + t) * 1024));
    dma16_lanes(m_src + (int64_t)j * 16, uniform(st + VG_AV + wave * VG_AM_LANES * 16), (1ull << VG_AM_LANES) - 1);
  };
  issue_a(0);

  // ---- table of gathered-row byte offsets for the whole reduction (this tile's V-row block) ----
  const uint32_t rowbytes = (uint32_t)(ldb * 2);
  for (int gi = tid; gi < KT * 16; gi += VG_NT) {
    const uint32_t sel4 = *reinterpret_cast<const uint32_t*>(colsel + 4 * (vblk * G + gi));
    const int s = gi >> 4, gg = gi & 15;
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = ((uint32_t)gi * (uint32_t)M + ((sel4 >> (8 * j)) & (uint32_t)(M - 1))) * rowbytes;
    *reinterpret_cast<u32x4*>(table + s * 64 + vg_tab_pos(4 * gg)) = o;
  }

  // ---- the wave's window of B: columns n0 + 64*wave .. +63 ----
  const int64_t wcol = n0 + 64 * wave;
  const int64_t b_bytes = ((G * M - 1) * ldb + Nc) * 2;   // first byte past the last element of B
  const int64_t w_off = wcol * 2 < b_bytes ? wcol * 2 : b_bytes;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)B + w_off), 0, (int)(b_bytes - w_off), 0x00020000);
  const uint32_t lane_col = 4u * (uint32_t)l32;

  // B of step kt into a register set: element h*16 + e' = the dword (columns 2c, 2c+1) of the
  // gathered row at table slot (h, hh, e').
  auto issue_b = [&](int kt, uint32_t (&b)[32]) {
    const uint32_t* tab = table + kt * 64 + 16 * hh;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(tab + 32 * h + 4 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[16 * h + 4 * q + j] = bload(t[j] + lane_col, rsrc);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][f][e] = 0.f;

  auto compute = [&](int kt, const uint32_t (&b)[32]) {
    const int s = kt & 1;
    const unsigned char* As = a_lds + ((kt >> 1) & 1) * VG_ASTAGE;
    const unsigned char* Ms = As + VG_AV;
    u32x2 mm[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) mm[i] = *reinterpret_cast<const u32x2*>(Ms + (32 * i + l32) * 16 + 8 * s);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 a[2];
      int idx[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 32 * i + l32;
        a[i] = *reinterpret_cast<const bf16x8*>(As + r * 128 + (vg_apos(r, 4 * s + 2 * h + hh) << 4));
        idx[i] = (int)(mm[i][h] >> (16 * hh));
      }
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint32_t sel = f ? 0x07060302u : 0x05040100u;
        u32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lo[q] = __builtin_amdgcn_perm(b[16 * h + 2 * q + 1], b[16 * h + 2 * q], sel);
          hi[q] = __builtin_amdgcn_perm(b[16 * h + 8 + 2 * q + 1], b[16 * h + 8 + 2 * q], sel);
        }
        const bf16x16 bop = __builtin_shufflevector(__builtin_bit_cast(bf16x8, lo), __builtin_bit_cast(bf16x8, hi), 0,
                                                    1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][f] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[i], bop, acc[i][f], idx[i], 0, 0);
      }
    }
  };

  // ---- pipeline ----
  // Issue order per wave: super-stage 0, then (after the table) B of steps 0 and 1; during even
  // step kt = 2j: super-stage j+1, then B of step kt+2; during odd step kt: B of step kt+2.
  // Loads complete in issue order, so before even step kt only B of step kt+1 (32 loads) may
  // still be outstanding (super-stage j was issued before B of step kt), and before odd step kt
  // super-stage j+1 and B of step kt+1 (32 + VG_LA).  Past the end, loads repeat the last step
  // or super-stage into a register set or buffer that is never read again.
  const int klast = KT - 1, jlast = KT / 2 - 1;
  uint32_t b0[32], b1[32], b2[32];
  lds_barrier();   // the table is complete
  issue_b(0, b0);
  issue_b(KT > 1 ? 1 : 0, b1);
  auto even = [&](int kt, uint32_t (&cur)[32], uint32_t (&nxt2)[32]) {
    wait_set<VG_LB>(cur);
    lds_barrier();   // super-stage kt/2 is in LDS for every wave; every wave is done with the other buffer
    const int j = kt >> 1;
    issue_a(j + 1 < jlast ? j + 1 : jlast);
    issue_b(kt + 2 < klast ? kt + 2 : klast, nxt2);
    compute(kt, cur);
  };
  auto odd = [&](int kt, uint32_t (&cur)[32], uint32_t (&nxt2)[32]) {
    wait_set<VG_LB + VG_LA>(cur);
    issue_b(kt + 2 < klast ? kt + 2 : klast, nxt2);
    compute(kt, cur);
  };
  for (int kt = 0;; kt += 6) {
    even(kt, b0, b2);
    odd(kt + 1, b1, b0);
    if (kt + 2 >= KT) break;
    even(kt + 2, b2, b1);
    odd(kt + 3, b0, b2);
    if (kt + 4 >= KT) break;
    even(kt + 4, b1, b0);
    odd(kt + 5, b2, b1);
    if (kt + 6 >= KT) break;
  }
  // drain: nothing may land in a register or in LDS after this point
  wait_set<0>(b0);
  wait_set<0>(b1);
  wait_set<0>(b2);

  // ---- epilogue: fragment f holds the columns of parity f, so (f = 0, f = 1) of one element is
  //      an 8-byte pair, and the 32 lanes of a row store 256 contiguous bytes ----
  const int64_t col = wcol + 2 * l32;
  if (col < Nc) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (row < R) {
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          const f32x2 o = {acc[i][0][e], acc[i][1][e]};
          __builtin_nontemporal_store(o, reinterpret_cast<f32x2*>(C + row * ldc + col));
        }
      }
    }
  }
}

// Conditions of the register-gather kernel beyond those of the row-major one: 64-row tiles inside
// one V-row block, the per-block table of gathered-row offsets in LDS next to two super-stages,
// B addressed with 32-bit offsets, 8-byte aligned pairs of C.
bool spmm_vnm_reg_ok(const uint8_t* colsel, int V, int M, int64_t G, int64_t Kd, int64_t ldb, int64_t Nc, const float* C,
                     int64_t ldc) {
  const int64_t lds = 2 * (int64_t)VG_ASTAGE + (Kd / 64) * VG_TAB_STEP;
  const int64_t b_bytes = ((G * M - 1) * ldb + Nc) * 2;
  return V % 64 == 0 && Kd % 128 == 0 && lds <= 64 * 1024 && b_bytes < ((int64_t)1 << 31) && Nc % 2 == 0 &&
         ldc % 2 == 0 && (uintptr_t)C % 8 == 0 && (uintptr_t)colsel % 4 == 0;
}

hipError_t launch_spmm_vnm_reg(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t Kd,
                               int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                               hipStream_t s) {
  const size_t lds = 2 * (size_t)VG_ASTAGE + (size_t)(Kd / 64) * VG_TAB_STEP;
  (void)hipFuncSetAttribute((const void*)spmm_vnm_reg_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t ntiles = ((R + VG_BM - 1) / VG_BM) * ((Nc + VG_BN - 1) / VG_BN);
  hipLaunchKernelGGL(spmm_vnm_reg_kernel, dim3((unsigned)ntiles), dim3(VG_NT), lds, s, (const uint16_t*)values, meta,
                     colsel, R, Kd, V, M, G, (const uint16_t*)B, ldb, Nc, C, ldc, 16);
  return hipGetLastError();
}

}  // namespace nms
