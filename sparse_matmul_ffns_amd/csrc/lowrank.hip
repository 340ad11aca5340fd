// Sparse weight plus a low-rank adapter, applied lazily (SLOPE abstract, NSF PAR award 2340011:
// low-rank adapters joined to the sparse weight for the last part of pre-training, with little
// extra cost in training and inference).
//
// The adapted weight W_s + U Vt (U [R][r], Vt [r][K]) is never formed.  The layer computes
//   Tt = Bt Vt^T           [Nc][r]  fp32: the adapter's inner activations, token-major
//   C  = W_s Bt^T + U Tt^T  [R][Nc]  fp32
// in two launches: lowrank_inner_kernel, then the K-contiguous 2:4 SpMM (spmm_nt.hip) with the
// adapter term added to its accumulators before they are stored.  Other shapes and fp32 take the
// plain SIMT kernels below after the general SpMM.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

namespace nms {

// Tt[n][j] = sum_k Bt[n][k] Vt[j][k] with bf16 operands and fp32 sums.  One workgroup per
// 32 x 32 block of Tt (32 rows of Bt, 32 rows of Vt), eight waves.  Both row blocks go to LDS by
// direct loads of whole 128-byte lines, in stages of 256 k (512-byte rows) through a ring of four
// buffers; the 16-byte chunk c of LDS row r holds source chunk c ^ (r % 16), so the operand reads
// of 16 consecutive rows hit distinct banks.  Wave w multiplies slices 2w and 2w+1 (16 k each) of
// every stage with v_mfma_f32_32x32x16_bf16 (A: Bt row n0 + l%32, k = 8*(l/32)..+7 of the slice;
// B: Vt row j0 + l%32, the same k).  The eight partial blocks are then added in LDS in a fixed
// tree order, so results do not depend on timing.
constexpr int kInnerStageK = 256;
constexpr int kInnerStages = 4;
constexpr int kInnerStageBytes = 64 * kInnerStageK * 2;   // 32 Bt rows + 32 Vt rows
constexpr int kInnerLds = kInnerStages * kInnerStageBytes;

__device__ __forceinline__ int inner_pos(int r, int c) { return c ^ (r & 15); }

__global__ __launch_bounds__(512) void lowrank_inner_kernel(const uint16_t* __restrict__ Bt, int64_t ldbt,
                                                            int64_t Nc, int64_t K, const uint16_t* __restrict__ Vt,
                                                            int64_t ldvt, int rank, float* __restrict__ Tt) {
  extern __shared__ __align__(1024) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, aa = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const int j0 = (int)blockIdx.y * 32;
  const uint32_t smem_base = lds_addr(smem);

  // stage st, 1 KB block b = 4*wave + q: Bt rows 2b, 2b+1 (b < 16) or Vt rows 2(b-16), 2(b-16)+1;
  // lane i -> row 2*(b % 16) + i/32, LDS chunk i % 32.  Chunks past K repeat the last one (never
  // read as operands).
  auto issue_stage = [&](int st, int64_t k0) {
    const int64_t left = (K - k0) / 8;
    const int nvalid = left < 32 ? (int)left : 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = 4 * wave + q;
      const int rr = 2 * (b & 15) + (lane >> 5);
      int c = inner_pos(rr, lane & 31);
      c = c < nvalid ? c : nvalid - 1;
      const uint32_t lds = uniform(smem_base + st * kInnerStageBytes + b * 1024);
      if (b < 16) {
        const int64_t n = n0 + rr < Nc ? n0 + rr : Nc - 1;
        dma16s((uint32_t)(2 * (n * ldbt + k0 + 8 * c)), Bt, lds);
      } else {
        const int64_t j = j0 + rr < rank ? j0 + rr : rank - 1;
        dma16s((uint32_t)(2 * (j * ldvt + k0 + 8 * c)), Vt, lds);
      }
    }
  };

  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  // a ring of four stage buffers: stage s is in buffer s % 4; while it is multiplied, the next
  // two are in flight and stage s + 3 is issued into the buffer stage s - 1 has left
  const int nst = (int)((K + kInnerStageK - 1) / kInnerStageK);
  for (int st = 0; st < 3 && st < nst; ++st) issue_stage(st, (int64_t)st * kInnerStageK);
  for (int st = 0; st < nst; ++st) {
    const int later = nst - 1 - st < 2 ? nst - 1 - st : 2;   // stages issued after this one
    if (later == 2) wait_vmcnt<8>();
    else if (later == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    lds_barrier();   // stage st is in LDS for every wave; every wave is done with stage st - 1
    if (st + 3 < nst) issue_stage((st + 3) % kInnerStages, (int64_t)(st + 3) * kInnerStageK);
    const unsigned char* S = smem + (st % kInnerStages) * kInnerStageBytes;
    const int64_t k0 = (int64_t)st * kInnerStageK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sl = 2 * wave + h;
      if (k0 + 16 * sl >= K) continue;
      const int c = 2 * sl + aa;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(S + l32 * 512 + (inner_pos(l32, c) << 4));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(S + 16384 + l32 * 512 + (inner_pos(l32, c) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  lds_barrier();   // every wave is done reading the stages before LDS is reused below

  // waves 4..7 hand their blocks to waves 0..3, then 2..3 to 0..1, then 1 to 0
  float* red = reinterpret_cast<float*>(smem);   // [4 slots][16 elements][64 lanes]
  for (int half = 4; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[((wave - half) * 16 + e) * 64 + lane] = acc[e];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += red[(wave * 16 + e) * 64 + lane];
    }
    __syncthreads();
  }
  const int j = j0 + l32;
  if (wave == 0 && j < rank) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = n0 + 8 * (e >> 2) + 4 * aa + (e & 3);
      if (row < Nc) Tt[row * rank + j] = acc[e];
    }
  }
}

// Plain SIMT forms (any shape, fp32 or bf16): one thread per output, sums in ascending k (j).
template <typename T>
__global__ __launch_bounds__(256) void lowrank_inner_generic_kernel(const T* __restrict__ Bt, int64_t ldbt, int64_t Nc,
                                                                    int64_t K, const T* __restrict__ Vt, int64_t ldvt,
                                                                    int rank, float* __restrict__ Tt) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Nc * rank) return;
  const int64_t n = idx / rank;
  const int64_t j = idx % rank;
  float s = 0.f;
  for (int64_t k = 0; k < K; ++k) s = fmaf(Elem<T>::to_f32(Bt[n * ldbt + k]), Elem<T>::to_f32(Vt[j * ldvt + k]), s);
  Tt[n * rank + j] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void lowrank_add_generic_kernel(const T* __restrict__ U, int64_t ldu,
                                                                  const float* __restrict__ Tt, int rank, int64_t R,
                                                                  int64_t Nc, float* __restrict__ C, int64_t ldc) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * Nc) return;
  const int64_t m = idx / Nc;
  const int64_t n = idx % Nc;
  float s = C[m * ldc + n];
  for (int j = 0; j < rank; ++j) s = fmaf(Elem<T>::to_f32(U[m * ldu + j]), Tt[n * rank + j], s);
  C[m * ldc + n] = s;
}

static bool al16(const void* p) { return (uintptr_t)p % 16 == 0; }

hipError_t launch_spmm_nm_t_lowrank(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                    const void* Bt, int64_t ldbt, int64_t Nc, const void* U, int64_t ldu,
                                    const void* Vt, int64_t ldvt, int64_t rank, float* Tt, float* C, int64_t ldc,
                                    hipStream_t s) {
  // Conditions of the matrix-instruction path: bf16, 16-wide adapter slices, 16-byte loads of Bt,
  // Vt, U and Tt rows, Bt and Vt addressable with 32-bit byte offsets.
  const bool fast = dt == DT_BF16 && !force_generic() && rank % 16 == 0 && K % 16 == 0 &&
                    ldbt % 8 == 0 && ldvt % 8 == 0 && ldu % 8 == 0 && al16(Bt) && al16(Vt) && al16(U) && al16(Tt) &&
                    Nc * ldbt * 2 < (int64_t(1) << 32) && rank * ldvt * 2 < (int64_t(1) << 32);
  hipError_t e;
  if (fast) {
    (void)hipFuncSetAttribute((const void*)lowrank_inner_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kInnerLds);
    const dim3 grid((unsigned)((Nc + 31) / 32), (unsigned)((rank + 31) / 32));
    hipLaunchKernelGGL(lowrank_inner_kernel, grid, dim3(512), (size_t)kInnerLds, s, (const uint16_t*)Bt, ldbt, Nc, K,
                       (const uint16_t*)Vt, ldvt, (int)rank, Tt);
    e = hipGetLastError();
  } else {
    const unsigned blocks = (unsigned)((Nc * rank + 255) / 256);
    if (dt == DT_BF16)
      hipLaunchKernelGGL(lowrank_inner_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)Bt,
                         ldbt, Nc, K, (const uint16_t*)Vt, ldvt, (int)rank, Tt);
    else
      hipLaunchKernelGGL(lowrank_inner_generic_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, (const uint32_t*)Bt,
                         ldbt, Nc, K, (const uint32_t*)Vt, ldvt, (int)rank, Tt);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  // the pipelined SpMM streams U and Tt into LDS with 32-bit byte offsets, like its other operands
  if (fast && spmm_nt_ok(values, meta, Bt, ldbt, R, Nc, K) && R * ldu * 2 < (int64_t(1) << 32) &&
      Nc * rank * 4 < (int64_t(1) << 32))
    return launch_spmm_nm_nt_dma_lowrank(values, meta, R, K, Bt, ldbt, Nc, U, ldu, Tt, (int)rank, C, ldc, s);
  e = launch_spmm_nm_t(dt, values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((R * Nc + 255) / 256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(lowrank_add_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)U, ldu, Tt,
                       (int)rank, R, Nc, C, ldc);
  else
    hipLaunchKernelGGL(lowrank_add_generic_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, (const uint32_t*)U, ldu, Tt,
                       (int)rank, R, Nc, C, ldc);
  return hipGetLastError();
}

}  // namespace nms
