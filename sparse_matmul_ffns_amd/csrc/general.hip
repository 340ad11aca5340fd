// General N:M SpMM with the dense operand K-contiguous: C = decompress(values, meta) Bt^T for any
// N:M form nm_compress writes (M in {4, 8, 16}, 1 <= N < M; "Success story: ESPLAG", Solution:
// N:M patterns beyond 2:4 in the VENOM format's family).
//
// When N <= 2 every aligned run of 4 columns holds at most two survivors, so the matrix is also a
// 2:4 matrix once each run is padded to two slots with +0.0: nm_to24_kernel rewrites the compressed
// form that way (into caller memory) and the 2:4 SMFMAC SpMM does the product at the 2:4 rate.
// With N > 2 a run can hold three or four survivors, which no structured-sparse matrix instruction
// takes; at those densities (3:4, 4:8, 6:8, ...) the matrix is expanded to dense bf16 rows in
// caller memory (nm_expand_kernel) and multiplied by the dense NT GEMM of the SDDMM
// (v_mfma_f32_32x32x16_bf16).  Other calls (fp32, or no work memory) take a plain SIMT kernel
// that decodes the position stream directly.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace nms {

// Fixed scratch memory for spmm_nm_general_noalloc: the 2:4 rewrite of the sparse operand lives
// here instead of in caller memory.  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it.  In host code `scratch` is only a stand-in for
// the device symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[GENERAL_SCRATCH_BYTES];

// b-bit field at bit offset bo of an LSB-first stream (the field never runs past its row).
__device__ inline uint32_t nm_field(const uint8_t* row, int64_t bo, int b) {
  const int64_t byte = bo >> 3;
  const int sh = (int)(bo & 7);
  uint32_t w = row[byte];
  if (sh + b > 8) w |= (uint32_t)row[byte + 1] << 8;
  return (w >> sh) & ((1u << b) - 1u);
}

// One thread per (row, output metadata byte): 2:4 runs q = 2t and 2t + 1 (dense columns 4q ..
// 4q+3) collect the survivors of their N:M group that fall inside them (at most two, in ascending
// position) and fill the remaining slots with +0.0 at the lowest free positions.
template <typename T>
__global__ __launch_bounds__(256) void nm_to24_kernel(const T* __restrict__ values, const uint8_t* __restrict__ meta,
                                                      int64_t R, int64_t K, int N, int M, T* __restrict__ v24,
                                                      uint8_t* __restrict__ m24) {
  // 32-bit index arithmetic (the launch guarantees R * ceil(K/8) < 2^32); M is a power of two
  const uint32_t tpr = (uint32_t)((K + 7) / 8);
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= (uint32_t)R * tpr) return;
  const uint32_t row = idx / tpr, t = idx - row * tpr;
  const int b = ceil_log2(M);
  const int64_t G = K >> b;
  const int64_t vrow = G * N, mrow = (G * N * b + 7) / 8;
  const uint8_t* mr = meta + row * mrow;
  uint32_t byte = 0;
  for (int h = 0; h < 2; ++h) {
    const int64_t q = 2 * (int64_t)t + h;
    if (4 * q >= K) break;
    const int64_t g = (4 * q) >> b;
    const int o = (int)(4 * q - (g << b));
    uint32_t p[2] = {0u, 1u};
    T v[2] = {T(0), T(0)};
    int cnt = 0;
    for (int s = 0; s < N; ++s) {
      const int pos = (int)nm_field(mr, (g * N + s) * b, b);
      if (pos >= o && pos < o + 4 && cnt < 2) {
        p[cnt] = (uint32_t)(pos - o);
        v[cnt] = values[row * vrow + g * N + s];
        ++cnt;
      }
    }
    if (cnt == 1) {   // one survivor: pair it with the lowest other position, holding +0.0
      if (p[0] == 0u) {
        p[1] = 1u;
        v[1] = T(0);
      } else {
        p[1] = p[0];
        v[1] = v[0];
        p[0] = 0u;
        v[0] = T(0);
      }
    }
    v24[(int64_t)row * (K / 2) + 2 * q] = v[0];
    v24[(int64_t)row * (K / 2) + 2 * q + 1] = v[1];
    byte |= (p[0] | (p[1] << 2)) << (4 * h);
  }
  m24[(int64_t)row * tpr + t] = (uint8_t)byte;
}

// The same rewrite for bf16 2:8 and 1:8 with 16-byte rows (K % 64 == 0): one thread per 24 bits of
// positions (4 groups of 2:8, 8 of 1:8), i.e. 8 kept values -- one 16-byte load of values, three
// byte loads of positions -- and 32 or 64 bytes of 2:4 values plus 4 or 8 bytes of nibbles out
// with 16-, 4- and 8-byte stores; consecutive threads cover consecutive bytes of every stream.  A
// group of 8 columns is the two runs 2g, 2g+1 of the 2:4 form, so its output nibble byte is g.
template <int N>
__global__ __launch_bounds__(256) void nm_to24_m8_kernel(const uint16_t* __restrict__ values,
                                                         const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                         uint16_t* __restrict__ v24, uint8_t* __restrict__ m24) {
  constexpr int GPT = N == 2 ? 4 : 8;   // groups per thread
  const uint32_t G = (uint32_t)(K / 8), per_row = G / GPT;
  const uint32_t u = blockIdx.x * 256u + threadIdx.x;
  if (u >= (uint32_t)R * per_row) return;
  const uint32_t r = u / per_row, q = u - r * per_row;
  const uint8_t* mp = meta + (int64_t)r * (3 * per_row) + 3 * q;
  const uint32_t bits = (uint32_t)mp[0] | ((uint32_t)mp[1] << 8) | ((uint32_t)mp[2] << 16);
  const u32x4 vin = *reinterpret_cast<const u32x4*>(values + (int64_t)r * G * N + (int64_t)q * GPT * N);
  uint32_t ov[2 * GPT];
  uint32_t ob[GPT];
#pragma unroll
  for (int g = 0; g < GPT; ++g) {
    uint32_t p[N], v[N];
#pragma unroll
    for (int s = 0; s < N; ++s) {
      const int i = g * N + s;   // survivor index within the thread's 8
      p[s] = (bits >> (3 * i)) & 7u;
      v[s] = (vin[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    }
    uint32_t nib[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // survivors inside run h (positions 4h .. 4h+3), in ascending position; free slots get +0.0
      // at the lowest free positions
      uint32_t cnt = 0, pa = 0, pb = 1, va = 0, vb = 0;
#pragma unroll
      for (int s = 0; s < N; ++s) {
        if ((p[s] >> 2) == (uint32_t)h) {
          if (cnt == 0) {
            pa = p[s] & 3u;
            va = v[s];
          } else {
            pb = p[s] & 3u;
            vb = v[s];
          }
          ++cnt;
        }
      }
      if (cnt == 1) {
        if (pa == 0) {
          pb = 1;
          vb = 0;
        } else {
          pb = pa;
          vb = va;
          pa = 0;
          va = 0;
        }
      }
      ov[2 * g + h] = va | (vb << 16);
      nib[h] = pa | (pb << 2);
    }
    ob[g] = nib[0] | (nib[1] << 4);
  }
  u32x4* vd = reinterpret_cast<u32x4*>(v24 + (int64_t)r * (K / 2) + (int64_t)q * GPT * 4);
#pragma unroll
  for (int k = 0; k < GPT / 2; ++k) vd[k] = u32x4{ov[4 * k], ov[4 * k + 1], ov[4 * k + 2], ov[4 * k + 3]};
  uint8_t* md = m24 + (int64_t)r * (K / 8) + (int64_t)q * GPT;
  if constexpr (GPT == 4) {
    *reinterpret_cast<uint32_t*>(md) = ob[0] | (ob[1] << 8) | (ob[2] << 16) | (ob[3] << 24);
  } else {
    *reinterpret_cast<u32x2*>(md) = u32x2{ob[0] | (ob[1] << 8) | (ob[2] << 16) | (ob[3] << 24),
                                          ob[4] | (ob[5] << 8) | (ob[6] << 16) | (ob[7] << 24)};
  }
}

// Dense bf16 rows of an N:M compressed matrix (the SpMM's own copy, row stride K): one thread per
// (row, group) reads the group's N values and N * log2(M) metadata bits, places each value at its
// position (a later survivor overwrites an earlier one at the same position, as nm_decompress
// does) and writes the group's M elements with one 8-, 16- or 32-byte store, so a wave's stores
// cover whole lines.  The group is held as M/4 64-bit words indexed by constant expressions.
template <int M>
__global__ __launch_bounds__(256) void nm_expand_kernel(const uint16_t* __restrict__ values,
                                                        const uint8_t* __restrict__ meta, int64_t R, int64_t K,
                                                        int N, uint16_t* __restrict__ out) {
  constexpr int b = M == 4 ? 2 : M == 8 ? 3 : 4;
  constexpr int W = M / 4;   // 64-bit words of a group
  const int64_t G = K / M;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= R * G) return;
  const int64_t r = u / G, g = u - r * G;
  const uint8_t* mr = meta + r * ((G * N * b + 7) / 8);
  const int64_t bit0 = g * N * b;
  const int sh = (int)(bit0 & 7);
  const int nb = (sh + N * b + 7) >> 3;   // at most 8 (N * b <= 60 and sh + N * b <= 64)
  uint64_t bits = 0;
  for (int i = 0; i < nb; ++i) bits |= (uint64_t)mr[(bit0 >> 3) + i] << (8 * i);
  bits >>= sh;
  const uint16_t* v = values + r * G * N + g * N;
  uint64_t w[W];
#pragma unroll
  for (int q = 0; q < W; ++q) w[q] = 0;
  for (int s = 0; s < N; ++s) {
    const uint32_t p = (uint32_t)(bits >> (s * b)) & (uint32_t)(M - 1);
    const uint32_t sft = 16 * (p & 3);
    const uint64_t put = (uint64_t)v[s] << sft, clr = ~((uint64_t)0xFFFF << sft);
#pragma unroll
    for (int q = 0; q < W; ++q)
      if ((p >> 2) == (uint32_t)q) w[q] = (w[q] & clr) | put;
  }
  uint16_t* o = out + r * K + g * M;
  if constexpr (W == 1) {
    *reinterpret_cast<uint64_t*>(o) = w[0];
  } else {
#pragma unroll
    for (int q = 0; q < W; q += 2)
      reinterpret_cast<u32x4*>(o)[q / 2] =
          u32x4{(uint32_t)w[q], (uint32_t)(w[q] >> 32), (uint32_t)w[q + 1], (uint32_t)(w[q + 1] >> 32)};
  }
}

// Plain SIMT product for any N:M (64 x 64 tiles, 32-k chunks staged densely in LDS): the kept
// values of each (row, group) are scattered to their dense columns by the decoded positions.
template <typename T>
__global__ __launch_bounds__(256) void spmm_general_generic_kernel(const T* __restrict__ values,
                                                                   const uint8_t* __restrict__ meta, int64_t R,
                                                                   int64_t K, int N, int M, const T* __restrict__ Bt,
                                                                   int64_t ldbt, int64_t Nc, float* __restrict__ C,
                                                                   int64_t ldc) {
  constexpr int TM = 64, TN = 64, KC = 32;
  __shared__ float As[KC][TM + 4];
  __shared__ float Bs[KC][TN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int b = ceil_log2(M);
  const int64_t G = K / M;
  const int64_t vrow = G * N, mrow = (G * N * b + 7) / 8;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    for (int i = tid; i < KC * TM; i += 256) As[i / TM][i % TM] = 0.f;
    __syncthreads();
    const int gpc = KC / M;   // M divides KC
    for (int u = tid; u < TM * gpc; u += 256) {
      const int r = u / gpc, gi = u % gpc;
      const int64_t row = m0 + r, g = k0 / M + gi;
      if (row >= R || g >= G) continue;
      for (int s = 0; s < N; ++s) {
        const uint32_t p = nm_field(meta + row * mrow, (g * N + s) * b, b) & (uint32_t)(M - 1);
        As[gi * M + p][r] = Elem<T>::to_f32(values[row * vrow + g * N + s]);
      }
    }
    for (int i = tid; i < KC * TN; i += 256) {
      const int kk = i % KC, nn = i / KC;
      const int64_t k = k0 + kk, n = n0 + nn;
      Bs[kk][nn] = (k < K && n < Nc) ? Elem<T>::to_f32(Bt[n * ldbt + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < KC; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= R) continue;
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n < Nc) C[row * ldc + n] = acc[i][j];
    }
  }
}

// Bytes of caller memory a route needs: the 2:4 rewrite (N <= 2: values [R][K/2], then metadata
// [R][ceil(K/8)] at the next 16-byte boundary) or the dense bf16 rows (N > 2, bf16, K % 64 == 0:
// [R][K]); 0 when the pattern takes neither.
int64_t general_work_bytes(int esz, int64_t R, int64_t K, int N, int M) {
  if (N == 2 && M == 4) return 0;
  if (N > 2) return esz == 2 && K % 64 == 0 ? R * K * 2 : 0;
  const int64_t vbytes = (R * (K / 2) * esz + 15) / 16 * 16;
  return vbytes + R * ((K + 7) / 8);
}

hipError_t launch_spmm_nm_general(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N, int M,
                                  const void* Bt, int64_t ldbt, int64_t Nc, float* C, int64_t ldc, void* work,
                                  int64_t work_bytes, hipStream_t s) {
  if (N == 2 && M == 4) return launch_spmm_nm_t(dt, values, meta, R, K, Bt, ldbt, Nc, C, ldc, s);
  const int esz = dt == DT_BF16 ? 2 : 4;
  const int64_t need = general_work_bytes(esz, R, K, N, M);
  if (N > 2 && need > 0 && work && work_bytes >= need && (uintptr_t)work % 16 == 0 && !force_generic() &&
      (R * (K / M) + 255) / 256 <= (int64_t)INT32_MAX &&
      dense_nt_fast_ok(work, K, Bt, ldbt, C, ldc, K)) {
    const int64_t groups = R * (K / M);
    const unsigned blocks = (unsigned)((groups + 255) / 256);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, (const uint16_t*)values, meta, R, K, N, (uint16_t*)work);
    };
    if (M == 4) go(nm_expand_kernel<4>);
    else if (M == 8) go(nm_expand_kernel<8>);
    else go(nm_expand_kernel<16>);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_dense_nt(work, K, Bt, ldbt, R, Nc, K, C, ldc, s);
  }
  if (N <= 2 && need > 0 && work && work_bytes >= need && (uintptr_t)work % 16 == 0 &&
      R * ((K + 7) / 8) < (int64_t(1) << 32) && !force_generic()) {
    unsigned char* w = (unsigned char*)work;
    uint8_t* m24 = w + (R * (K / 2) * esz + 15) / 16 * 16;
    const unsigned blocks = (unsigned)((R * ((K + 7) / 8) + 255) / 256);
    if (dt == DT_BF16 && M == 8 && K % 64 == 0 && (uintptr_t)values % 16 == 0) {
      // 2:8 and 1:8: one thread per 8 kept values (4 groups of 2:8, 8 of 1:8)
      const int64_t threads = R * (K / (N == 2 ? 32 : 64));
      const unsigned b2 = (unsigned)((threads + 255) / 256);
      if (N == 2)
        hipLaunchKernelGGL(nm_to24_m8_kernel<2>, dim3(b2), dim3(256), 0, s, (const uint16_t*)values, meta, R, K,
                           (uint16_t*)w, m24);
      else
        hipLaunchKernelGGL(nm_to24_m8_kernel<1>, dim3(b2), dim3(256), 0, s, (const uint16_t*)values, meta, R, K,
                           (uint16_t*)w, m24);
    } else if (dt == DT_BF16)
      hipLaunchKernelGGL(nm_to24_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)values, meta, R, K,
                         N, M, (uint16_t*)w, m24);
    else
      hipLaunchKernelGGL(nm_to24_kernel<uint32_t>, dim3(blocks), dim3(256), 0, s, (const uint32_t*)values, meta, R, K,
                         N, M, (uint32_t*)w, m24);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_spmm_nm_t(dt, w, m24, R, K, Bt, ldbt, Nc, C, ldc, s);
  }
  const dim3 grid((unsigned)((Nc + 63) / 64), (unsigned)((R + 63) / 64));
  if (dt == DT_BF16)
    hipLaunchKernelGGL(spmm_general_generic_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)values, meta, R,
                       K, N, M, (const uint16_t*)Bt, ldbt, Nc, C, ldc);
  else
    hipLaunchKernelGGL(spmm_general_generic_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)values, meta, R,
                       K, N, M, (const uint32_t*)Bt, ldbt, Nc, C, ldc);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per device (with that device
// current) and cached.
static hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// spmm_nm_general with the 2:4 rewrite in `scratch`: the same kernels, no allocation.  Returns
// hipErrorInvalidValue (before any launch) when the rewrite needs more than GENERAL_SCRATCH_BYTES;
// the caller checks that first.  Nothing in `scratch` has to start at zero: the rewrite writes every
// byte the product reads.
hipError_t launch_spmm_nm_general_noalloc(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                          int N, int M, const void* Bt, int64_t ldbt, int64_t Nc, float* C,
                                          int64_t ldc, hipStream_t s) {
  const int64_t need = general_work_bytes(dt == DT_BF16 ? 2 : 4, R, K, N, M);
  if (need > GENERAL_SCRATCH_BYTES) return hipErrorInvalidValue;
  void* ptr = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ptr);
    if (e != hipSuccess) return e;
  }
  return launch_spmm_nm_general(dt, values, meta, R, K, N, M, Bt, ldbt, Nc, C, ldc, ptr, need, s);
}

}  // namespace nms
