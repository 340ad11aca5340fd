// Host-side launchers of the gfx950 kernels (internal to libnmsparse).
// Arguments are validated by api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nms {

enum { DT_F32 = 0, DT_BF16 = 1 };

inline int64_t meta_row_bytes(int64_t K, int N, int M) {
  int b = 1;
  while ((1 << b) < M) ++b;
  return ((K / M) * N * b + 7) / 8;
}

hipError_t launch_nm_prune(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                           uint8_t* mask, int64_t ldmask, hipStream_t s);
hipError_t launch_nm_compress(int dt, const void* A, int64_t lda, const uint8_t* mask, int64_t ldmask,
                              int64_t R, int64_t K, int N, int M, void* values, uint8_t* meta, int32_t* bad,
                              hipStream_t s);
hipError_t launch_nm_prune_compress(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                    uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta, hipStream_t s);
hipError_t launch_nm_prune_compress_transpose(int dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                              uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta,
                                              const void* B, int64_t ldb, int64_t KB, int64_t Nc, void* Bt,
                                              int64_t ldbt, hipStream_t s);
hipError_t launch_nm_decompress(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N,
                                int M, void* out, int64_t lda, hipStream_t s);
hipError_t launch_prune_act_venom(int dt, const void* Z, int64_t ldz, int64_t R, int64_t K, int V, int M,
                                  int relu, void* values, uint8_t* meta, uint8_t* colsel, uint8_t* mask,
                                  int64_t ldmask, hipStream_t s);
hipError_t launch_nm_reprune_t(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                               void* values_t, uint8_t* meta_t, hipStream_t s);
hipError_t launch_nm_reprune_t_transpose(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                         void* values_t, uint8_t* meta_t, const void* X, int64_t ldx, int64_t RX,
                                         int64_t CX, void* Xt, int64_t ldxt, hipStream_t s);
hipError_t launch_spmm_nm(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                          int64_t ldb, int64_t Nc, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_venom(int dt, const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                             int64_t K, int V, int M, const void* B, int64_t ldb, int64_t Nc, float* C,
                             int64_t ldc, hipStream_t s);
bool spmm_dma_ok(const void* values, const uint8_t* meta, const void* B, int64_t ldb, int64_t Nc, int64_t Kd);
hipError_t launch_spmm_nm_dma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                              int64_t ldb, int64_t Nc, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_venom_dma(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                                 int64_t Kd, int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc,
                                 float* C, int64_t ldc, hipStream_t s);
bool spmm_vnm_reg_ok(const uint8_t* colsel, int V, int M, int64_t G, int64_t Kd, int64_t ldb, int64_t Nc, const float* C,
                     int64_t ldc);
hipError_t launch_spmm_vnm_reg(const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R, int64_t Kd,
                               int V, int M, int64_t G, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                               hipStream_t s);
bool spmm_nt_ok(const void* values, const uint8_t* meta, const void* Bt, int64_t ldbt, int64_t R, int64_t Nc,
                int64_t Kd);
hipError_t launch_spmm_nm_t(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                            int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_nt_dma(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                 int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_nt_dma_bf16out(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                         int64_t ldbt, int64_t Nc, uint16_t* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_t_bf16out(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                   const void* Bt, int64_t ldbt, int64_t Nc, uint16_t* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_nt_dma_lowrank(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                         int64_t ldbt, int64_t Nc, const void* U, int64_t ldu, const float* Tt,
                                         int rank, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_t_lowrank(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                    const void* Bt, int64_t ldbt, int64_t Nc, const void* U, int64_t ldu,
                                    const void* Vt, int64_t ldvt, int64_t rank, float* Tt, float* C, int64_t ldc,
                                    hipStream_t s);
hipError_t launch_spmm_nm_t_relu_venom(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                      int64_t ldbt, int64_t Nc, int V, int M, void* hv, uint8_t* hm, uint8_t* hc,
                                      hipStream_t s);
int64_t general_work_bytes(int esz, int64_t R, int64_t K, int N, int M);
// Size of the fixed scratch memory of spmm_nm_general_noalloc (64 MiB per GPU).
constexpr int64_t GENERAL_SCRATCH_BYTES = int64_t(64) << 20;
hipError_t launch_spmm_nm_general_noalloc(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                          int N, int M, const void* Bt, int64_t ldbt, int64_t Nc, float* C,
                                          int64_t ldc, hipStream_t s);
hipError_t launch_spmm_nm_general(int dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N, int M,
                                  const void* Bt, int64_t ldbt, int64_t Nc, float* C, int64_t ldc, void* work,
                                  int64_t work_bytes, hipStream_t s);
hipError_t launch_nm_transpose(int dt, const void* src, int64_t lds, int64_t R, int64_t Cn, void* dst, int64_t ldd,
                               hipStream_t s);
bool spmm_panels_ok(const void* values, const uint8_t* meta, const void* Bt, int64_t ldbt, int64_t R, int64_t K,
                    int64_t Nc);
hipError_t launch_spmm_nm_t_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                                   int64_t ldbt, int64_t Nc, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_nm_reprune_t_transpose_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                                void* values_t, uint8_t* meta_t, const void* X, int64_t ldx,
                                                int64_t RX, int64_t CX, void* Xt, int64_t ldxt, hipStream_t s);
hipError_t launch_nm_to_panels(const void* values, const uint8_t* meta, int64_t R, int64_t K, void* values_p,
                               uint8_t* meta_p, hipStream_t s);
int64_t mfma_probe_flops(int kind, int64_t iters);
hipError_t launch_mfma_rate_probe(int kind, int64_t iters, float* sink, hipStream_t s);
hipError_t launch_sddmm_nm_dt(int dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                              int64_t Tn, const uint8_t* meta, float* out, void* Dt, int64_t lddt, hipStream_t s);
bool sddmm_venom_fast_ok(const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn, int64_t F, int64_t Nc,
                         int V, int M, const void* hv, const float* dz, const void* dYt, int64_t lddyt);
hipError_t launch_sddmm_venom_dma(const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn, int64_t F,
                                  int64_t Nc, int V, int M, const void* hv, const uint8_t* hm, const uint8_t* hc,
                                  int relu, float* dz, void* dYt, int64_t lddyt, hipStream_t s);
bool dense_nt_fast_ok(const void* A, int64_t lda, const void* B, int64_t ldb, const float* out, int64_t ldo,
                      int64_t Tn);
hipError_t launch_dense_nt(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t R, int64_t Kc, int64_t Tn,
                           float* out, int64_t ldo, hipStream_t s);
int64_t venom_tn_work_bytes(int esz, int64_t Tn, int64_t F);
hipError_t launch_sddmm_venom(int dt, const void* dY, int64_t lddy, const void* Wd, int64_t ldw, int64_t Tn,
                              int64_t F, int64_t Nc, int V, int M, const void* hv, const uint8_t* hm,
                              const uint8_t* hc, int relu, float* dz, void* dYt, int64_t lddyt, hipStream_t s);
hipError_t launch_spmm_venom_tn(int dt, const void* hv, const uint8_t* hm, const uint8_t* hc, int64_t Tn, int64_t F,
                                int V, int M, const void* dYt, int64_t lddyt, int64_t Nc, float* dW, int64_t lddw,
                                void* work, int64_t work_bytes, hipStream_t s);
hipError_t launch_sddmm_nm(int dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R,
                           int64_t Kc, int64_t T, const uint8_t* meta, float* out, hipStream_t s);

}  // namespace nms
