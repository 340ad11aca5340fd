// C ABI of libnmsparse: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is launched; a call that
// returns an error has touched no device memory.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../include/nmsparse.h"
#include "launch.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

nm_status hip_status(hipError_t e) {
  if (e == hipSuccess) return NM_OK;
  const char* s = hipGetErrorString(e);
  strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return NM_ERR_HIP;
}

bool dtype_ok(nm_dtype dt) { return dt == NM_F32 || dt == NM_BF16; }
int esize(nm_dtype dt) { return dt == NM_BF16 ? 2 : 4; }
bool aligned(const void* p, int a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }
bool m_ok(int M) { return M == 4 || M == 8 || M == 16; }
bool nm_ok(int N, int M) { return m_ok(M) && N >= 1 && N < M; }
bool v_ok(int V) { return V >= 1 && V <= 256; }
hipStream_t hs(nm_stream s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

nm_status nm_prune(nm_dtype dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M, uint8_t* mask,
                   int64_t ldmask, nm_stream stream) {
  if (!A || !mask) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || K % M != 0 || lda < K || ldmask < K) return NM_ERR_SHAPE;
  if (!aligned(A, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_prune(dt, A, lda, R, K, N, M, mask, ldmask, hs(stream)));
}

nm_status nm_compress(nm_dtype dt, const void* A, int64_t lda, const uint8_t* mask, int64_t ldmask, int64_t R,
                      int64_t K, int N, int M, void* values, uint8_t* meta, int32_t* bad_groups,
                      nm_stream stream) {
  if (!A || !mask || !values || !meta) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || K % M != 0 || lda < K || ldmask < K) return NM_ERR_SHAPE;
  if (!aligned(A, esize(dt)) || !aligned(values, esize(dt)) || !aligned(bad_groups, 4)) return NM_ERR_ALIGN;
  return hip_status(
      nms::launch_nm_compress(dt, A, lda, mask, ldmask, R, K, N, M, values, meta, bad_groups, hs(stream)));
}

nm_status nm_prune_compress(nm_dtype dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                            uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta, nm_stream stream) {
  if (!A || !mask || !values || !meta) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || K % M != 0 || lda < K || ldmask < K) return NM_ERR_SHAPE;
  if (!aligned(A, esize(dt)) || !aligned(values, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_prune_compress(dt, A, lda, R, K, N, M, mask, ldmask, values, meta, hs(stream)));
}

nm_status nm_prune_compress_transpose(nm_dtype dt, const void* A, int64_t lda, int64_t R, int64_t K, int N, int M,
                                      uint8_t* mask, int64_t ldmask, void* values, uint8_t* meta, const void* B,
                                      int64_t ldb, int64_t KB, int64_t Nc, void* Bt, int64_t ldbt, nm_stream stream) {
  if (!A || !mask || !values || !meta || !B || !Bt) return NM_ERR_NULL;
  if (dt != NM_BF16 || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || K % M != 0 || lda < K || ldmask < K) return NM_ERR_SHAPE;
  if (KB <= 0 || Nc <= 0 || ldb < Nc || ldbt < KB) return NM_ERR_SHAPE;
  if (!aligned(A, esize(dt)) || !aligned(values, esize(dt)) || !aligned(B, esize(dt)) || !aligned(Bt, esize(dt)))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_prune_compress_transpose(dt, A, lda, R, K, N, M, mask, ldmask, values, meta, B,
                                                            ldb, KB, Nc, Bt, ldbt, hs(stream)));
}

nm_status nm_decompress(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N, int M,
                        void* A_out, int64_t lda, nm_stream stream) {
  if (!values || !meta || !A_out) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || K % M != 0 || lda < K) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(A_out, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_decompress(dt, values, meta, R, K, N, M, A_out, lda, hs(stream)));
}

nm_status spmm_nm(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* B,
                  int64_t ldb, int64_t Nc, float* C, int64_t ldc, nm_stream stream) {
  if (!values || !meta || !B || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % 4 != 0 || ldb < Nc || ldc < Nc) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(B, esize(dt)) || !aligned(C, 4)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_nm(dt, values, meta, R, K, B, ldb, Nc, C, ldc, hs(stream)));
}

nm_status spmm_nm_t(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                    int64_t ldbt, int64_t Nc, float* C, int64_t ldc, nm_stream stream) {
  if (!values || !meta || !Bt || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % 4 != 0 || ldbt < K || ldc < Nc) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(Bt, esize(dt)) || !aligned(C, 4)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_nm_t(dt, values, meta, R, K, Bt, ldbt, Nc, C, ldc, hs(stream)));
}

nm_status spmm_nm_t_out_bf16(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                             const void* Bt, int64_t ldbt, int64_t Nc, void* C, int64_t ldc, nm_stream stream) {
  if (!values || !meta || !Bt || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % 4 != 0 || ldbt < K || ldc < Nc) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(Bt, esize(dt)) || !aligned(C, 2)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_nm_t_bf16out(dt, values, meta, R, K, Bt, ldbt, Nc, (uint16_t*)C, ldc,
                                                  hs(stream)));
}

nm_status spmm_nm_t_lowrank(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                            const void* Bt, int64_t ldbt, int64_t Nc, const void* U, int64_t ldu, const void* Vt,
                            int64_t ldvt, int64_t rank, float* Tt, float* C, int64_t ldc, nm_stream stream) {
  if (!values || !meta || !Bt || !U || !Vt || !Tt || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || rank <= 0 || rank > (1 << 20) || K % 4 != 0 || ldbt < K || ldc < Nc ||
      ldu < rank || ldvt < K)
    return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(Bt, esize(dt)) || !aligned(U, esize(dt)) || !aligned(Vt, esize(dt)) ||
      !aligned(Tt, 4) || !aligned(C, 4))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_nm_t_lowrank(dt, values, meta, R, K, Bt, ldbt, Nc, U, ldu, Vt, ldvt, rank, Tt, C,
                                                  ldc, hs(stream)));
}

nm_status spmm_nm_general(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N, int M,
                          const void* Bt, int64_t ldbt, int64_t Nc, float* C, int64_t ldc, void* work,
                          int64_t work_bytes, nm_stream stream) {
  if (!values || !meta || !Bt || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % M != 0 || ldbt < K || ldc < Nc || work_bytes < 0) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(Bt, esize(dt)) || !aligned(C, 4)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_nm_general(dt, values, meta, R, K, N, M, Bt, ldbt, Nc, C, ldc, work, work_bytes,
                                                hs(stream)));
}

nm_status spmm_nm_general_noalloc(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, int N,
                                  int M, const void* Bt, int64_t ldbt, int64_t Nc, float* C, int64_t ldc,
                                  nm_stream stream) {
  if (!values || !meta || !Bt || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !nm_ok(N, M)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % M != 0 || ldbt < K || ldc < Nc) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(Bt, esize(dt)) || !aligned(C, 4)) return NM_ERR_ALIGN;
  if (nms::general_work_bytes(esize(dt), R, K, N, M) > nms::GENERAL_SCRATCH_BYTES) return NM_ERR_TOO_LARGE;
  return hip_status(nms::launch_spmm_nm_general_noalloc(dt, values, meta, R, K, N, M, Bt, ldbt, Nc, C, ldc,
                                                        hs(stream)));
}

nm_status sddmm_venom(nm_dtype dt, const void* dY, int64_t lddy, const void* W_down, int64_t ldw, int64_t T,
                      int64_t F, int64_t Nc, int V, int M, const void* h_values, const uint8_t* h_meta,
                      const uint8_t* h_colsel, int apply_relu, float* dz, void* dYt, int64_t lddyt,
                      nm_stream stream) {
  if (!dY || !W_down || !h_values || !h_meta || !h_colsel || !dz) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !m_ok(M) || !v_ok(V) || (dYt && dt != NM_BF16)) return NM_ERR_UNSUPPORTED;
  if (T <= 0 || F <= 0 || Nc <= 0 || F % M != 0 || T % V != 0 || lddy < Nc || ldw < Nc || (dYt && lddyt < T))
    return NM_ERR_SHAPE;
  if (!aligned(dY, esize(dt)) || !aligned(W_down, esize(dt)) || !aligned(h_values, 2 * esize(dt)) ||
      !aligned(h_colsel, 4) || !aligned(dz, 8) || !aligned(dYt, esize(dt)))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_sddmm_venom(dt, dY, lddy, W_down, ldw, T, F, Nc, V, M, h_values, h_meta, h_colsel,
                                            apply_relu ? 1 : 0, dz, dYt, lddyt, hs(stream)));
}

nm_status spmm_venom_tn(nm_dtype dt, const void* h_values, const uint8_t* h_meta, const uint8_t* h_colsel, int64_t T,
                        int64_t F, int V, int M, const void* dYt, int64_t lddyt, int64_t Nc, float* dW, int64_t lddw,
                        void* work, int64_t work_bytes, nm_stream stream) {
  if (!h_values || !h_meta || !h_colsel || !dYt || !dW) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !m_ok(M) || !v_ok(V)) return NM_ERR_UNSUPPORTED;
  if (T <= 0 || F <= 0 || Nc <= 0 || F % M != 0 || T % V != 0 || lddyt < T || lddw < Nc || work_bytes < 0)
    return NM_ERR_SHAPE;
  if (!aligned(h_values, 2 * esize(dt)) || !aligned(h_colsel, 4) || !aligned(dYt, esize(dt)) || !aligned(dW, 4))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_spmm_venom_tn(dt, h_values, h_meta, h_colsel, T, F, V, M, dYt, lddyt, Nc, dW, lddw,
                                              work, work_bytes, hs(stream)));
}

int64_t nm_venom_tn_work_bytes(nm_dtype dt, int64_t T, int64_t F) {
  if (!dtype_ok(dt) || T <= 0 || F <= 0) return 0;
  return nms::venom_tn_work_bytes(esize(dt), T, F);
}

int nm_gmp_n_at(int M, int n_final, int64_t t_begin, int64_t t_end, int64_t interval, int64_t t_dense, int64_t step,
                int* prune_now) {
  if (prune_now) *prune_now = 0;
  if (!m_ok(M) || n_final < 1 || n_final >= M || t_begin < 0 || t_end < t_begin || interval < 1) return -1;
  if (step < t_begin || (t_dense >= 0 && step >= t_dense)) return M;   // dense before the ramp and after the switch
  const int64_t events = (t_end - t_begin) / interval + 1;           // at t_begin + e * interval
  int64_t e = (step - t_begin) / interval;                             // the last event at or before step
  if (e > events - 1) e = events - 1;
  if (prune_now && (step - t_begin) % interval == 0 && (step - t_begin) / interval < events) *prune_now = 1;
  const int64_t removed = ((int64_t)(M - n_final) * (e + 1) + events - 1) / events;   // ceil
  return M - (int)removed;
}

int64_t nm_general_scratch_bytes(void) { return nms::GENERAL_SCRATCH_BYTES; }

int64_t nm_general_work_bytes(nm_dtype dt, int64_t R, int64_t K, int N, int M) {
  if (!dtype_ok(dt) || !nm_ok(N, M) || R <= 0 || K <= 0 || K % M != 0) return 0;
  return nms::general_work_bytes(esize(dt), R, K, N, M);
}

nm_status spmm_nm_t_relu_venom(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                               const void* Bt, int64_t ldbt, int64_t Nc, int V, int M, void* h_values,
                               uint8_t* h_meta, uint8_t* h_colsel, nm_stream stream) {
  if (!values || !meta || !Bt || !h_values || !h_meta || !h_colsel) return NM_ERR_NULL;
  if (dt != NM_BF16 || (V != 64 && V != 128 && V != 256) || (M != 4 && M != 8 && M != 16)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || K % 4 != 0 || ldbt < K || R % M != 0 || Nc % V != 0) return NM_ERR_SHAPE;
  if (!aligned(values, 2) || !aligned(Bt, 2) || !aligned(h_values, 2)) return NM_ERR_ALIGN;
  const hipError_t e = nms::launch_spmm_nm_t_relu_venom(values, meta, R, K, Bt, ldbt, Nc, V, M, h_values, h_meta,
                                                        h_colsel, hs(stream));
  if (e == hipErrorNotSupported) return NM_ERR_UNSUPPORTED;
  return hip_status(e);
}

nm_status nm_transpose(nm_dtype dt, const void* src, int64_t lds, int64_t R, int64_t Cn, void* dst, int64_t ldd,
                       nm_stream stream) {
  if (!src || !dst) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || Cn <= 0 || lds < Cn || ldd < R) return NM_ERR_SHAPE;
  if (!aligned(src, esize(dt)) || !aligned(dst, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_transpose(dt, src, lds, R, Cn, dst, ldd, hs(stream)));
}

nm_status prune_act_venom(nm_dtype dt, const void* Z, int64_t ldz, int64_t R, int64_t K, int V, int M,
                          int apply_relu, void* values, uint8_t* meta, uint8_t* colsel, uint8_t* mask,
                          int64_t ldmask, nm_stream stream) {
  if (!Z || !values || !meta || !colsel) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !m_ok(M) || !v_ok(V)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || R % V != 0 || K % M != 0 || ldz < K || (mask && ldmask < K)) return NM_ERR_SHAPE;
  if (!aligned(Z, esize(dt)) || !aligned(values, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_prune_act_venom(dt, Z, ldz, R, K, V, M, apply_relu != 0, values, meta, colsel,
                                                mask, ldmask, hs(stream)));
}

nm_status spmm_venom(nm_dtype dt, const void* values, const uint8_t* meta, const uint8_t* colsel, int64_t R,
                     int64_t K, int V, int M, const void* B, int64_t ldb, int64_t Nc, float* C, int64_t ldc,
                     nm_stream stream) {
  if (!values || !meta || !colsel || !B || !C) return NM_ERR_NULL;
  if (!dtype_ok(dt) || !m_ok(M) || !v_ok(V)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || R % V != 0 || K % M != 0 || ldb < Nc || ldc < Nc) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(B, esize(dt)) || !aligned(C, 4)) return NM_ERR_ALIGN;
  return hip_status(
      nms::launch_spmm_venom(dt, values, meta, colsel, R, K, V, M, B, ldb, Nc, C, ldc, hs(stream)));
}

nm_status nm_reprune_t(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, void* values_t,
                       uint8_t* meta_t, nm_stream stream) {
  if (!values || !meta || !values_t || !meta_t) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || R % 4 != 0 || K % 4 != 0) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(values_t, esize(dt))) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_reprune_t(dt, values, meta, R, K, values_t, meta_t, hs(stream)));
}

nm_status nm_reprune_t_transpose(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                 void* values_t, uint8_t* meta_t, const void* X, int64_t ldx, int64_t RX, int64_t CX,
                                 void* Xt, int64_t ldxt, nm_stream stream) {
  if (!values || !meta || !values_t || !meta_t || !X || !Xt) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || R % 4 != 0 || K % 4 != 0) return NM_ERR_SHAPE;
  if (RX <= 0 || CX <= 0 || ldx < CX || ldxt < RX) return NM_ERR_SHAPE;
  if (!aligned(values, esize(dt)) || !aligned(values_t, esize(dt)) || !aligned(X, esize(dt)) || !aligned(Xt, esize(dt)))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_reprune_t_transpose(dt, values, meta, R, K, values_t, meta_t, X, ldx, RX, CX, Xt,
                                                       ldxt, hs(stream)));
}

nm_status nm_mfma_rate_probe(int kind, int64_t iters, float* sink, int64_t* flops, nm_stream stream) {
  if (!sink || !flops) return NM_ERR_NULL;
  if (kind != 0 && kind != 1) return NM_ERR_UNSUPPORTED;
  if (iters <= 0 || iters > (int64_t(1) << 24)) return NM_ERR_SHAPE;
  if (!aligned(sink, 4)) return NM_ERR_ALIGN;
  *flops = nms::mfma_probe_flops(kind, iters);
  return hip_status(nms::launch_mfma_rate_probe(kind, iters, sink, hs(stream)));
}

nm_status nm_to_panels(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, void* values_p,
                       uint8_t* meta_p, nm_stream stream) {
  if (!values || !meta || !values_p || !meta_p) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || R % 4 != 0 || K % 256 != 0) return NM_ERR_SHAPE;
  if (!aligned(values, 16) || !aligned(meta, 16) || !aligned(values_p, 16) || !aligned(meta_p, 16)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_to_panels(values, meta, R, K, values_p, meta_p, hs(stream)));
}

nm_status nm_reprune_t_transpose_panels(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K,
                                        void* values_t, uint8_t* meta_t, const void* X, int64_t ldx, int64_t RX,
                                        int64_t CX, void* Xt, int64_t ldxt, nm_stream stream) {
  if (!values || !meta || !values_t || !meta_t || !X || !Xt) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || R % 256 != 0 || K % 128 != 0) return NM_ERR_SHAPE;
  if (RX <= 0 || CX <= 0 || ldx < CX || ldxt < RX) return NM_ERR_SHAPE;
  if (!aligned(values, 16) || !aligned(meta, 2) || !aligned(values_t, 16) || !aligned(meta_t, 2) ||
      !aligned(X, esize(dt)) || !aligned(Xt, esize(dt)))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_nm_reprune_t_transpose_panels(values, meta, R, K, values_t, meta_t, X, ldx, RX, CX, Xt,
                                                              ldxt, hs(stream)));
}

nm_status spmm_nm_t_panels(nm_dtype dt, const void* values, const uint8_t* meta, int64_t R, int64_t K, const void* Bt,
                           int64_t ldbt, int64_t Nc, float* C, int64_t ldc, nm_stream stream) {
  if (!values || !meta || !Bt || !C) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || K <= 0 || Nc <= 0 || R % 256 != 0 || K % 256 != 0 || ldbt < K || ldbt % 8 != 0 || ldc < Nc)
    return NM_ERR_SHAPE;
  if (!aligned(values, 16) || !aligned(meta, 16) || !aligned(Bt, 16) || !aligned(C, 4)) return NM_ERR_ALIGN;
  if (R * K >= (int64_t(1) << 32) || Nc * ldbt * 2 >= (int64_t(1) << 32)) return NM_ERR_TOO_LARGE;
  const hipError_t e = nms::launch_spmm_nm_t_panels(values, meta, R, K, Bt, ldbt, Nc, C, ldc, hs(stream));
  if (e == hipErrorNotSupported) return NM_ERR_UNSUPPORTED;
  return hip_status(e);
}

nm_status sddmm_nm(nm_dtype dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                   int64_t T, const uint8_t* meta, float* values_out, nm_stream stream) {
  if (!D || !X || !meta || !values_out) return NM_ERR_NULL;
  if (!dtype_ok(dt)) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || Kc <= 0 || T <= 0 || Kc % 4 != 0 || ldd < T || ldx < T) return NM_ERR_SHAPE;
  if (!aligned(D, esize(dt)) || !aligned(X, esize(dt)) || !aligned(values_out, 4)) return NM_ERR_ALIGN;
  return hip_status(nms::launch_sddmm_nm(dt, D, ldd, X, ldx, R, Kc, T, meta, values_out, hs(stream)));
}

nm_status sddmm_nm_dt(nm_dtype dt, const void* D, int64_t ldd, const void* X, int64_t ldx, int64_t R, int64_t Kc,
                      int64_t T, const uint8_t* meta, float* values_out, void* Dt, int64_t lddt, nm_stream stream) {
  if (!D || !X || !meta || !values_out || !Dt) return NM_ERR_NULL;
  if (dt != NM_BF16) return NM_ERR_UNSUPPORTED;
  if (R <= 0 || Kc <= 0 || T <= 0 || Kc % 4 != 0 || ldd < T || ldx < T || lddt < R) return NM_ERR_SHAPE;
  if (!aligned(D, esize(dt)) || !aligned(X, esize(dt)) || !aligned(values_out, 4) || !aligned(Dt, esize(dt)))
    return NM_ERR_ALIGN;
  return hip_status(nms::launch_sddmm_nm_dt(dt, D, ldd, X, ldx, R, Kc, T, meta, values_out, Dt, lddt, hs(stream)));
}

void nm_sizes(int64_t R, int64_t K, int N, int M, int V, int64_t* n_values, int64_t* meta_bytes,
              int64_t* colsel_bytes) {
  if (M <= 0) M = 4;
  const int64_t G = K / M;
  if (V > 0) {
    if (n_values) *n_values = R * G * 2;
    if (meta_bytes) *meta_bytes = R * ((G + 1) / 2);
    if (colsel_bytes) *colsel_bytes = (R / V) * G * 4;
  } else {
    if (n_values) *n_values = R * G * N;
    if (meta_bytes) *meta_bytes = R * nms::meta_row_bytes(K, N, M);
    if (colsel_bytes) *colsel_bytes = 0;
  }
}

const char* nm_status_str(nm_status status) {
  switch (status) {
    case NM_OK: return "ok";
    case NM_ERR_NULL: return "a required pointer is NULL";
    case NM_ERR_SHAPE: return "invalid shape or leading dimension";
    case NM_ERR_UNSUPPORTED: return "unsupported dtype, N:M pattern or block size";
    case NM_ERR_ALIGN: return "pointer not aligned to its element size";
    case NM_ERR_HIP: return "HIP launch failed";
    case NM_ERR_TOO_LARGE: return "the operand needs more scratch memory than the library's fixed buffer holds";
  }
  return "unknown status";
}

const char* nm_last_hip_error(void) { return g_last_hip_error; }

int nm_version(void) { return 100; }

}  // extern "C"
