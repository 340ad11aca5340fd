// The matrix-core rate the chip sustains (gfx950): a chip-wide loop of independent matrix
// instructions on register operands, no memory traffic.  Under such a load the chip lowers its
// clock to stay within its power limit, so this rate -- not the nominal 2.4 GHz one -- is what a
// matrix-bound kernel can approach.  Measurement aid only: no step of the sparse path calls it.
#include "common.hpp"
#include "launch.hpp"

namespace nms {

// KIND 0: v_mfma_f32_32x32x16_bf16 (dense); KIND 1: v_smfmac_f32_32x32x32_bf16 (2:4).  Each wave
// keeps 8 independent accumulators (no instruction waits for the previous one's result).  The
// operands change every iteration -- random signs and significands from a per-lane linear
// congruential sequence, exponents near 1 -- because the power a matrix instruction draws, and
// with it the clock the chip can hold, depends on how many operand bits toggle: with constant
// operands the loop runs near the nominal rate.  One value per lane is written at the end, so
// nothing is optimised away.
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(int64_t iters, float* __restrict__ sink) {
  uint32_t x = 0x9E3779B9u * (uint32_t)(blockIdx.x * 256 + threadIdx.x + 1);
  const int idx = 0x4E4E4E4E;   // per group nibble p0 | p1 << 2 = 2 | 3 << 2 or 0 | 1 << 2: valid 2:4
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
    x = x * 1664525u + 1013904223u;
    u32x4 av;
    uint32_t bw[8];
    // bf16 pairs: random sign and significand bits, exponent 0x7E or 0x7F (magnitudes 0.5 .. 2)
#pragma unroll
    for (int k = 0; k < 4; ++k) av[k] = ((x ^ (0x85EBCA6Bu * (uint32_t)(k + 1))) & 0x80FF80FFu) | 0x3F003F00u;
#pragma unroll
    for (int k = 0; k < 8; ++k) bw[k] = ((x ^ (0xC2B2AE35u * (uint32_t)(k + 1))) & 0x80FF80FFu) | 0x3F003F00u;
    const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND == 0) {
        const u32x4 b4 = {bw[(j & 1) * 4], bw[(j & 1) * 4 + 1], bw[(j & 1) * 4 + 2], bw[(j & 1) * 4 + 3]};
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b4), acc[j], 0, 0, 0);
      } else {
        typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
        const u32x8 b8 = {bw[0], bw[1], bw[2], bw[3], bw[4], bw[5], bw[6], bw[7]};
        acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, __builtin_bit_cast(bf16x16, b8), acc[j], idx, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid: two workgroups of four waves per CU (two waves per SIMD) on 256 CUs.
constexpr int kProbeBlocks = 512;

int64_t mfma_probe_flops(int kind, int64_t iters) {
  const int64_t per_instr = kind == 0 ? 2LL * 32 * 32 * 16 : 2LL * 32 * 32 * 32;   // dense-equivalent
  return per_instr * 8 * iters * (int64_t)kProbeBlocks * 4;
}

hipError_t launch_mfma_rate_probe(int kind, int64_t iters, float* sink, hipStream_t s) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(kProbeBlocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(kProbeBlocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace nms
