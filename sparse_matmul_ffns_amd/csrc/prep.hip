// The two streaming passes that prepare a 2:4 FFN product in one launch (gfx950):
// nm_prune_compress of the weight A and nm_transpose of the activations B.  They touch
// disjoint data, and each alone is a short HBM-bound kernel that spends part of its time filling
// and draining the chip; one grid with the transpose's workgroups first and the prune's after
// them keeps HBM busy across both (18.7 us against 21.1 us for the two launches at
// A [8192 x 2048], B [2048 x 4096]).  Every workgroup runs exactly the code of the kernel it
// stands for (prep_bodies.hpp), so the outputs are those of the two calls.
#include "common.hpp"
#include "launch.hpp"
#include "prep_bodies.hpp"

namespace nms {

__global__ __launch_bounds__(256) void prune_compress_transpose_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t R, int64_t K, uint8_t* __restrict__ mask, int64_t ldmask,
    uint16_t* __restrict__ values, uint8_t* __restrict__ meta, const uint16_t* __restrict__ B, int64_t ldb,
    int64_t KB, int64_t Nc, uint16_t* __restrict__ Bt, int64_t ldbt, int n_transpose) {
  const int b = blockIdx.x;
  if (b < n_transpose)
    transpose_bf16_body(b, B, ldb, KB, Nc, Bt, ldbt);
  else
    prune_compress24_body<uint16_t, uint32_t, kPrepU>(b - n_transpose, A, lda, R, K, mask, ldmask, values, meta);
}

hipError_t launch_nm_prune_compress_transpose(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                              uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta,
                                              const void* B, int64_t ldb, int64_t KB, int64_t Nc, void* Bt,
                                              int64_t ldbt, hipStream_t s) {
  const int64_t n = R * (K / 16);   // 16-element chunks of A
  const bool fused = dt == DT_BF16 && N == 2 && M == 4 && K % 16 == 0 && (uintptr_t)A % 16 == 0 &&
                     (lda * 2) % 16 == 0 && (uintptr_t)mask % 16 == 0 && ldmask % 16 == 0 &&
                     (uintptr_t)values % 16 == 0 && (uintptr_t)meta % 2 == 0 &&
                     n + 256 * kPrepU < (int64_t)UINT32_MAX;
  if (!fused) {   // the two calls, each with its own paths
    const hipError_t e = launch_nm_prune_compress(dt, A, lda, R, K, N, M, mask, ldmask, values, meta, s);
    if (e != hipSuccess) return e;
    return launch_nm_transpose(dt, B, ldb, KB, Nc, Bt, ldbt, s);
  }
  const int64_t n_prune = (n + 256 * kPrepU - 1) / (256 * kPrepU);
  const int64_t tiles = ((KB + 63) / 64) * ((Nc + 63) / 64);
  const int64_t n_transpose = (tiles + 3) / 4;
  if (n_prune + n_transpose > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prune_compress_transpose_kernel, dim3((unsigned)(n_prune + n_transpose)), dim3(256), 0, s,
                     (const uint16_t*)A, lda, R, K, mask, ldmask, (uint16_t*)values, meta, (const uint16_t*)B, ldb,
                     KB, Nc, (uint16_t*)Bt, ldbt, (int)n_transpose);
  return hipGetLastError();
}

}  // namespace nms
