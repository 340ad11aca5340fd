// Host-side exercise of every libnmsparse entry point, built with AddressSanitizer on the host
// code of the C ABI (tests/test_host_asan.py builds and runs it on a machine without a GPU).
// Invalid arguments must return their documented status before any launch; valid arguments
// with placeholder device addresses pass validation and reach the launcher, which reports the
// missing device (NM_ERR_HIP).  ASan reports any out-of-bounds or use-after-free access of the
// host code on the way.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nmsparse.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                   \
  do {                                                                                       \
    const int got_ = (int)(expr);                                                            \
    if (got_ != (int)(want)) {                                                               \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, (int)(want)); \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

int main() {
  // placeholder device addresses, 256-byte aligned, never dereferenced on the host
  void* P = (void*)(uintptr_t)0x10000;
  uint8_t* U8 = (uint8_t*)P;
  float* F = (float*)P;
  int32_t* I32 = (int32_t*)P;
  const nm_dtype B = NM_BF16, S = NM_F32;
  const nm_status H = NM_ERR_HIP;   // valid arguments, no device

  // nm_prune / nm_compress / nm_prune_compress / nm_prune_compress_transpose / nm_decompress
  EXPECT(nm_prune(B, P, 8, 4, 8, 2, 4, U8, 8, 0), H);
  EXPECT(nm_prune(B, NULL, 8, 4, 8, 2, 4, U8, 8, 0), NM_ERR_NULL);
  EXPECT(nm_prune(B, P, 8, 4, 10, 2, 4, U8, 10, 0), NM_ERR_SHAPE);
  EXPECT(nm_prune(B, P, 8, 4, 8, 3, 5, U8, 8, 0), NM_ERR_UNSUPPORTED);
  EXPECT(nm_prune(S, (char*)P + 2, 8, 4, 8, 2, 4, U8, 8, 0), NM_ERR_ALIGN);
  EXPECT(nm_compress(B, P, 16, U8, 16, 4, 16, 2, 8, P, U8, I32, 0), H);
  EXPECT(nm_compress(B, P, 16, U8, 16, 4, 16, 2, 8, P, NULL, I32, 0), NM_ERR_NULL);
  EXPECT(nm_prune_compress(S, P, 16, 4, 16, 4, 16, U8, 16, P, U8, 0), H);
  EXPECT(nm_prune_compress(S, P, 8, 4, 16, 4, 16, U8, 16, P, U8, 0), NM_ERR_SHAPE);
  EXPECT(nm_prune_compress_transpose(B, P, 64, 64, 64, 2, 4, U8, 64, P, U8, P, 64, 64, 64, P, 64, 0), H);
  EXPECT(nm_decompress(B, P, U8, 4, 8, 2, 4, P, 8, 0), H);
  EXPECT(nm_decompress(B, P, U8, 4, 8, 2, 4, P, 4, 0), NM_ERR_SHAPE);

  // products
  EXPECT(spmm_nm(B, P, U8, 64, 128, P, 64, 64, F, 64, 0), H);
  EXPECT(spmm_nm(B, P, U8, 64, 128, P, 32, 64, F, 64, 0), NM_ERR_SHAPE);
  EXPECT(spmm_nm_t(B, P, U8, 64, 256, P, 256, 64, F, 64, 0), H);
  EXPECT(spmm_nm_t_out_bf16(B, P, U8, 64, 256, P, 256, 64, P, 64, 0), H);
  EXPECT(spmm_nm_t_lowrank(B, P, U8, 64, 256, P, 256, 64, P, 64, P, 256, 64, F, F, 64, 0), H);
  EXPECT(spmm_nm_t_relu_venom(B, P, U8, 256, 256, P, 256, 256, 128, 8, P, U8, U8, 0), H);
  EXPECT(spmm_nm_t_relu_venom(B, P, U8, 264, 256, P, 256, 256, 128, 8, P, U8, U8, 0), NM_ERR_UNSUPPORTED);
  EXPECT(spmm_nm_general(B, P, U8, 64, 128, 2, 8, P, 128, 64, F, 64, P, 1 << 20, 0), H);
  EXPECT(spmm_nm_general(B, P, U8, 64, 128, 2, 8, P, 128, 64, F, 64, NULL, -1, 0), NM_ERR_SHAPE);
  EXPECT(spmm_nm_general_noalloc(B, P, U8, 64, 128, 2, 8, P, 128, 64, F, 64, 0), H);
  EXPECT(spmm_nm_general_noalloc(B, P, U8, 65536, 1024, 2, 8, P, 1024, 8, F, 8, 0), NM_ERR_TOO_LARGE);
  EXPECT(nm_transpose(B, P, 64, 64, 64, P, 64, 0), H);
  EXPECT(prune_act_venom(B, P, 64, 128, 64, 128, 8, 1, P, U8, U8, NULL, 0, 0), H);
  EXPECT(prune_act_venom(B, P, 64, 100, 64, 128, 8, 1, P, U8, U8, NULL, 0, 0), NM_ERR_SHAPE);
  EXPECT(spmm_venom(B, P, U8, U8, 128, 256, 64, 8, P, 64, 64, F, 64, 0), H);
  EXPECT(spmm_venom(B, P, U8, U8, 128, 256, 0, 8, P, 64, 64, F, 64, 0), NM_ERR_UNSUPPORTED);
  EXPECT(nm_reprune_t(B, P, U8, 128, 128, P, U8, 0), H);
  EXPECT(nm_reprune_t(B, P, U8, 126, 128, P, U8, 0), NM_ERR_SHAPE);
  EXPECT(nm_reprune_t_transpose(B, P, U8, 128, 128, P, U8, P, 64, 64, 64, P, 64, 0), H);
  EXPECT(nm_reprune_t_transpose(B, P, U8, 128, 128, P, U8, P, 32, 64, 64, P, 64, 0), NM_ERR_SHAPE);
  EXPECT(nm_reprune_t_transpose(S, P, U8, 128, 128, P, U8, P, 64, 64, 64, P, 64, 0), NM_ERR_UNSUPPORTED);
  EXPECT(sddmm_nm(B, P, 64, P, 64, 64, 64, 64, U8, F, 0), H);
  EXPECT(sddmm_nm_dt(B, P, 64, P, 64, 64, 64, 64, U8, F, P, 64, 0), H);
  EXPECT(sddmm_venom(B, P, 64, P, 64, 128, 256, 64, 128, 8, P, U8, U8, 1, F, P, 128, 0), H);
  EXPECT(sddmm_venom(B, P, 64, P, 64, 100, 256, 64, 128, 8, P, U8, U8, 1, F, NULL, 0, 0), NM_ERR_SHAPE);
  EXPECT(spmm_venom_tn(B, P, U8, U8, 128, 256, 64, 8, P, 128, 64, F, 64, P, 1 << 20, 0), H);
  EXPECT(spmm_venom_tn(B, P, U8, U8, 128, 256, 64, 8, P, 64, 64, F, 64, NULL, 0, 0), NM_ERR_SHAPE);

  // host-only helpers
  int64_t nv = -1, mb = -1, cb = -1;
  nm_sizes(8192, 16384, 2, 8, 128, &nv, &mb, &cb);
  EXPECT(nv == 8192 * 4096 && mb == 8192 * 1024 && cb == 64 * 2048 * 4, 1);
  nm_sizes(8, 16, 2, 4, 0, &nv, &mb, NULL);
  EXPECT(nm_general_work_bytes(B, 8, 64, 2, 8), 8 * 32 * 2 + 8 * 8);
  EXPECT(nm_venom_tn_work_bytes(B, 64, 128), 64 * 128 * 2);
  EXPECT(nm_general_scratch_bytes() == (int64_t)64 << 20, 1);
  int ev = -1;
  EXPECT(nm_gmp_n_at(8, 2, 2, 8, 3, 12, 5, &ev), 4);
  EXPECT(ev, 1);
  EXPECT(nm_gmp_n_at(8, 2, 2, 8, 3, 12, 13, NULL), 8);
  for (int s = 0; s <= 7; ++s) EXPECT(nm_status_str((nm_status)s) != NULL && strlen(nm_status_str((nm_status)s)) > 1, 1);
  EXPECT(strlen(nm_last_hip_error()) > 0, 1);   // the last valid call above failed to launch
  EXPECT(nm_version() >= 100, 1);

  if (failures) return 1;
  printf("asan abi ok\n");
  return 0;
}
