"""The C ABI loads, exports every declared symbol and rejects bad arguments
before launching anything (CPU only: no call here reaches a kernel)."""

import ctypes

import pytest

from sparse_matmul_ffns_amd import nmsparse as nm

FAKE = 4096  # a non-NULL address that is never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    return nm.lib()


def test_exports_every_header_function(L):
    names = nm.header_functions()
    assert set(names) >= {"nm_prune", "nm_compress", "spmm_nm", "spmm_venom", "prune_act_venom",
                          "nm_decompress", "nm_reprune_t", "sddmm_nm", "nm_sizes", "nm_status_str"}
    for name in names:
        assert hasattr(L, name), name


def test_binding_covers_header():
    assert set(nm._SIGNATURES) | {"nm_sizes", "nm_status_str", "nm_last_hip_error", "nm_version",
                                  "nm_general_work_bytes", "nm_general_scratch_bytes",
                                  "nm_venom_tn_work_bytes", "nm_gmp_n_at"} == set(nm.header_functions())


def test_status_strings(L):
    for s in range(7):
        assert L.nm_status_str(s) and L.nm_status_str(s) != b"unknown status"
    assert L.nm_version() >= 100
    assert L.nm_last_hip_error() == b""


def test_sizes():
    assert nm.sizes(8192, 2048, 2, 4) == (8192 * 1024, 8192 * 256, 0)
    assert nm.sizes(3, 12, 2, 4) == (18, 3 * 2, 0)                  # ceil(12/8) = 2 bytes per row
    assert nm.sizes(2, 16, 2, 8) == (8, 2 * 2, 0)                   # 4 fields x 3 bits -> 2 bytes
    assert nm.sizes(8192, 16384, 2, 8, 128) == (8192 * 4096, 8192 * 1024, 64 * 2048 * 4)
    assert nm.sizes(4, 24, 2, 8, 2) == (4 * 6, 4 * 2, 2 * 3 * 4)    # 3 groups -> 2 bytes of nibbles


def test_prune_errors(L):
    s = None
    assert L.nm_prune(1, None, 8, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.nm_prune(1, FAKE, 8, 4, 8, 2, 4, None, 8, s) == nm.NM_ERR_NULL
    assert L.nm_prune(7, FAKE, 8, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_prune(1, FAKE, 8, 4, 8, 2, 5, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_prune(1, FAKE, 8, 4, 8, 4, 4, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_prune(1, FAKE, 8, 4, 8, 0, 4, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_prune(1, FAKE, 8, 0, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_SHAPE
    assert L.nm_prune(1, FAKE, 8, 4, 10, 2, 4, FAKE, 10, s) == nm.NM_ERR_SHAPE   # K % M
    assert L.nm_prune(1, FAKE, 4, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_SHAPE     # lda < K
    assert L.nm_prune(1, FAKE, 8, 4, 8, 2, 4, FAKE, 7, s) == nm.NM_ERR_SHAPE     # ldmask < K
    assert L.nm_prune(1, FAKE + 1, 8, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_ALIGN
    assert L.nm_prune(0, FAKE + 2, 8, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_ALIGN


def test_compress_decompress_errors(L):
    s = None
    assert L.nm_compress(1, FAKE, 8, FAKE, 8, 4, 8, 2, 4, None, FAKE, None, s) == nm.NM_ERR_NULL
    assert L.nm_compress(1, FAKE, 8, FAKE, 8, 4, 8, 2, 16, FAKE, FAKE, None, s) == nm.NM_ERR_SHAPE
    assert L.nm_compress(1, FAKE, 8, FAKE, 8, 4, 8, 2, 4, FAKE + 1, FAKE, None, s) == nm.NM_ERR_ALIGN
    assert L.nm_compress(1, FAKE, 8, FAKE, 8, 4, 8, 2, 4, FAKE, FAKE, FAKE + 2, s) == nm.NM_ERR_ALIGN
    assert L.nm_decompress(1, FAKE, None, 4, 8, 2, 4, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.nm_decompress(1, FAKE, FAKE, 4, 8, 2, 4, FAKE, 6, s) == nm.NM_ERR_SHAPE
    assert L.nm_decompress(1, FAKE, FAKE, 4, 8, 3, 3, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED


def test_spmm_errors(L):
    s = None
    assert L.spmm_nm(1, FAKE, FAKE, 4, 8, None, 8, 8, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.spmm_nm(1, FAKE, FAKE, 4, 6, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE       # K % 4
    assert L.spmm_nm(1, FAKE, FAKE, 4, 8, FAKE, 4, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE       # ldb < Nc
    assert L.spmm_nm(1, FAKE, FAKE, 4, 8, FAKE, 8, 8, FAKE, 7, s) == nm.NM_ERR_SHAPE       # ldc < Nc
    assert L.spmm_nm(1, FAKE, FAKE, 4, 8, FAKE, 8, 0, FAKE, 8, s) == nm.NM_ERR_SHAPE
    assert L.spmm_nm(3, FAKE, FAKE, 4, 8, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.spmm_nm(1, FAKE, FAKE, 4, 8, FAKE, 8, 8, FAKE + 2, 8, s) == nm.NM_ERR_ALIGN
    assert L.spmm_venom(1, FAKE, FAKE, None, 4, 16, 2, 8, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.spmm_venom(1, FAKE, FAKE, FAKE, 4, 16, 3, 8, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE  # R % V
    assert L.spmm_venom(1, FAKE, FAKE, FAKE, 4, 16, 2, 6, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.spmm_venom(1, FAKE, FAKE, FAKE, 4, 16, 0, 8, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.spmm_venom(1, FAKE, FAKE, FAKE, 512, 16, 512, 8, FAKE, 8, 8, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED


def test_venom_reprune_sddmm_errors(L):
    s = None
    assert L.prune_act_venom(1, FAKE, 16, 4, 16, 2, 8, 1, FAKE, FAKE, None, None, 0, s) == nm.NM_ERR_NULL
    assert L.prune_act_venom(1, FAKE, 16, 4, 12, 2, 8, 1, FAKE, FAKE, FAKE, None, 0, s) == nm.NM_ERR_SHAPE
    assert L.prune_act_venom(1, FAKE, 16, 4, 16, 2, 8, 1, FAKE, FAKE, FAKE, FAKE, 8, s) == nm.NM_ERR_SHAPE
    assert L.prune_act_venom(1, FAKE, 16, 4, 16, 257, 8, 1, FAKE, FAKE, FAKE, None, 0, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_reprune_t(1, FAKE, FAKE, 6, 8, FAKE, FAKE, s) == nm.NM_ERR_SHAPE
    assert L.nm_reprune_t(1, FAKE, FAKE, 8, 8, FAKE, None, s) == nm.NM_ERR_NULL
    assert L.nm_reprune_t(1, FAKE, FAKE, 8, 8, FAKE + 1, FAKE, s) == nm.NM_ERR_ALIGN
    # nm_reprune_t_transpose(dt, values, meta, R, K, values_t, meta_t, X, ldx, RX, CX, Xt, ldxt, stream)
    assert L.nm_reprune_t_transpose(1, FAKE, FAKE, 8, 8, FAKE, FAKE, None, 8, 8, 8, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.nm_reprune_t_transpose(0, FAKE, FAKE, 8, 8, FAKE, FAKE, FAKE, 8, 8, 8, FAKE, 8, s) == \
        nm.NM_ERR_UNSUPPORTED
    assert L.nm_reprune_t_transpose(1, FAKE, FAKE, 6, 8, FAKE, FAKE, FAKE, 8, 8, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE
    assert L.nm_reprune_t_transpose(1, FAKE, FAKE, 8, 8, FAKE, FAKE, FAKE, 4, 8, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE
    assert L.nm_reprune_t_transpose(1, FAKE, FAKE, 8, 8, FAKE, FAKE, FAKE, 8, 8, 8, FAKE, 4, s) == nm.NM_ERR_SHAPE
    assert L.nm_reprune_t_transpose(1, FAKE, FAKE, 8, 8, FAKE, FAKE, FAKE + 1, 8, 8, 8, FAKE, 8, s) == \
        nm.NM_ERR_ALIGN
    assert L.sddmm_nm(1, FAKE, 8, FAKE, 8, 4, 6, 8, FAKE, FAKE, s) == nm.NM_ERR_SHAPE
    assert L.sddmm_nm(1, FAKE, 4, FAKE, 8, 4, 8, 8, FAKE, FAKE, s) == nm.NM_ERR_SHAPE
    assert L.sddmm_nm(1, FAKE, 8, FAKE, 8, 4, 8, 8, None, FAKE, s) == nm.NM_ERR_NULL
    assert L.sddmm_nm(1, FAKE, 8, FAKE, 8, 4, 8, 8, FAKE, FAKE + 2, s) == nm.NM_ERR_ALIGN


def test_lowrank_general_fused_errors(L):
    s = None
    # spmm_nm_t_lowrank(dt, values, meta, R, K, Bt, ldbt, Nc, U, ldu, Vt, ldvt, rank, Tt, C, ldc, stream)
    assert L.spmm_nm_t_lowrank(1, FAKE, FAKE, 8, 16, FAKE, 16, 8, FAKE, 16, FAKE, 16, 16, None, FAKE, 8, s) == \
        nm.NM_ERR_NULL
    assert L.spmm_nm_t_lowrank(1, FAKE, FAKE, 8, 16, FAKE, 16, 8, FAKE, 8, FAKE, 16, 16, FAKE, FAKE, 8, s) == \
        nm.NM_ERR_SHAPE                                                                      # ldu < rank
    assert L.spmm_nm_t_lowrank(1, FAKE, FAKE, 8, 16, FAKE, 16, 8, FAKE, 16, FAKE, 16, 0, FAKE, FAKE, 8, s) == \
        nm.NM_ERR_SHAPE                                                                      # rank 0
    assert L.spmm_nm_t_lowrank(1, FAKE, FAKE, 8, 16, FAKE, 16, 8, FAKE + 1, 16, FAKE, 16, 16, FAKE, FAKE, 8, s) == \
        nm.NM_ERR_ALIGN
    # spmm_nm_general(dt, values, meta, R, K, N, M, Bt, ldbt, Nc, C, ldc, work, work_bytes, stream)
    assert L.spmm_nm_general(1, FAKE, FAKE, 8, 16, 2, 5, FAKE, 16, 8, FAKE, 8, None, 0, s) == nm.NM_ERR_UNSUPPORTED
    assert L.spmm_nm_general(1, FAKE, FAKE, 8, 12, 2, 8, FAKE, 16, 8, FAKE, 8, None, 0, s) == nm.NM_ERR_SHAPE
    assert L.spmm_nm_general(1, FAKE, FAKE, 8, 16, 2, 8, FAKE, 16, 8, FAKE, 8, None, -1, s) == nm.NM_ERR_SHAPE
    assert L.spmm_nm_general(1, None, FAKE, 8, 16, 2, 8, FAKE, 16, 8, FAKE, 8, None, 0, s) == nm.NM_ERR_NULL
    assert L.nm_general_work_bytes(1, 8, 64, 2, 8) == 8 * 32 * 2 + 8 * 8
    assert L.nm_general_work_bytes(0, 8, 64, 1, 4) == 8 * 32 * 4 + 8 * 8
    assert L.nm_general_work_bytes(1, 8, 64, 3, 8) == 8 * 64 * 2
    assert L.nm_general_work_bytes(0, 8, 64, 3, 8) == 0
    assert L.nm_general_work_bytes(1, 8, 72, 3, 8) == 0
    # sddmm_venom(dt, dY, lddy, Wd, ldw, T, F, Nc, V, M, hv, hm, hc, relu, dz, dYt, lddyt, stream)
    assert L.sddmm_venom(1, None, 8, FAKE, 8, 128, 64, 8, 128, 8, FAKE, FAKE, FAKE, 1, FAKE, None, 0, s) == \
        nm.NM_ERR_NULL
    assert L.sddmm_venom(1, FAKE, 8, FAKE, 8, 128, 64, 8, 128, 6, FAKE, FAKE, FAKE, 1, FAKE, None, 0, s) == \
        nm.NM_ERR_UNSUPPORTED
    assert L.sddmm_venom(0, FAKE, 8, FAKE, 8, 128, 64, 8, 128, 8, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 128, s) == \
        nm.NM_ERR_UNSUPPORTED                                  # dY^T only in bf16
    assert L.sddmm_venom(1, FAKE, 8, FAKE, 8, 100, 64, 8, 128, 8, FAKE, FAKE, FAKE, 1, FAKE, None, 0, s) == \
        nm.NM_ERR_SHAPE                                        # T % V
    assert L.sddmm_venom(1, FAKE, 8, FAKE, 8, 128, 64, 8, 128, 8, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 64, s) == \
        nm.NM_ERR_SHAPE                                        # lddyt < T
    assert L.sddmm_venom(1, FAKE + 2, 8, FAKE, 8, 128, 64, 8, 128, 8, FAKE, FAKE, FAKE, 1, FAKE + 4, None, 0, s) == \
        nm.NM_ERR_ALIGN                                        # dz not 8-byte aligned
    # spmm_venom_tn(dt, hv, hm, hc, T, F, V, M, dYt, lddyt, Nc, dW, lddw, work, work_bytes, stream)
    assert L.spmm_venom_tn(1, FAKE, FAKE, None, 128, 64, 128, 8, FAKE, 128, 8, FAKE, 8, None, 0, s) == \
        nm.NM_ERR_NULL
    assert L.spmm_venom_tn(1, FAKE, FAKE, FAKE, 128, 60, 128, 8, FAKE, 128, 8, FAKE, 8, None, 0, s) == \
        nm.NM_ERR_SHAPE                                        # F % M
    assert L.spmm_venom_tn(1, FAKE, FAKE, FAKE, 128, 64, 128, 8, FAKE, 128, 8, FAKE, 8, None, -1, s) == \
        nm.NM_ERR_SHAPE
    assert L.nm_venom_tn_work_bytes(1, 8192, 16384) == 8192 * 16384 * 2
    assert L.nm_venom_tn_work_bytes(0, 64, 64) == 0
    # spmm_nm_general_noalloc(dt, values, meta, R, K, N, M, Bt, ldbt, Nc, C, ldc, stream)
    assert L.nm_general_scratch_bytes() == 64 << 20
    assert L.spmm_nm_general_noalloc(1, None, FAKE, 8, 16, 2, 8, FAKE, 16, 8, FAKE, 8, s) == nm.NM_ERR_NULL
    assert L.spmm_nm_general_noalloc(1, FAKE, FAKE, 8, 16, 2, 5, FAKE, 16, 8, FAKE, 8, s) == nm.NM_ERR_UNSUPPORTED
    assert L.spmm_nm_general_noalloc(1, FAKE, FAKE, 8, 12, 2, 8, FAKE, 16, 8, FAKE, 8, s) == nm.NM_ERR_SHAPE
    # a 2:8 matrix whose 2:4 rewrite (R*K/2 bf16 + R*K/8 bytes) exceeds 64 MiB: rejected before any launch
    big_r, big_k = 65536, 1024
    assert L.nm_general_work_bytes(1, big_r, big_k, 2, 8) > L.nm_general_scratch_bytes()
    assert L.spmm_nm_general_noalloc(1, FAKE, FAKE, big_r, big_k, 2, 8, FAKE, big_k, 8, FAKE, 8, s) == \
        nm.NM_ERR_TOO_LARGE
    # spmm_nm_t_relu_venom(dt, values, meta, R, K, Bt, ldbt, Nc, V, M, hv, hm, hc, stream)
    assert L.spmm_nm_t_relu_venom(1, FAKE, FAKE, 256, 256, FAKE, 256, 256, 128, 8, FAKE, None, FAKE, s) == \
        nm.NM_ERR_NULL
    assert L.spmm_nm_t_relu_venom(0, FAKE, FAKE, 256, 256, FAKE, 256, 256, 128, 8, FAKE, FAKE, FAKE, s) == \
        nm.NM_ERR_UNSUPPORTED                                                                # fp32
    assert L.spmm_nm_t_relu_venom(1, FAKE, FAKE, 256, 256, FAKE, 256, 256, 32, 8, FAKE, FAKE, FAKE, s) == \
        nm.NM_ERR_UNSUPPORTED                                                                # V = 32
    assert L.spmm_nm_t_relu_venom(1, FAKE, FAKE, 256, 256, FAKE, 256, 200, 128, 8, FAKE, FAKE, FAKE, s) == \
        nm.NM_ERR_SHAPE                                                                      # Nc % V
    assert L.spmm_nm_t_relu_venom(1, FAKE, FAKE, 264, 256, FAKE, 256, 256, 128, 8, FAKE, FAKE, FAKE, s) == \
        nm.NM_ERR_UNSUPPORTED                                                                # R % 256: no fused tile


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nm.nm_prune(torch.zeros(4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        nm.spmm_nm(torch.zeros(4, 4, dtype=torch.bfloat16), torch.zeros(4, 1, dtype=torch.uint8), 8,
                   torch.zeros(8, 8, dtype=torch.bfloat16))


# gradual pruning schedules worked by hand from the stated rule (events at t_begin + e*interval,
# N_e = M - ceil((M - n_final)(e + 1)/E), dense before t_begin and from t_dense on)
GMP_HAND = [
    # (M, n_final, t_begin, t_end, interval, t_dense): [(step, N, pruning event)]
    ((8, 2, 2, 8, 3, 12), [(0, 8, 0), (1, 8, 0), (2, 6, 1), (3, 6, 0), (4, 6, 0), (5, 4, 1), (6, 4, 0), (7, 4, 0),
                           (8, 2, 1), (9, 2, 0), (11, 2, 0), (12, 8, 0), (40, 8, 0)]),
    ((4, 2, 0, 0, 1, -1), [(0, 2, 1), (1, 2, 0), (1000, 2, 0)]),
    ((16, 1, 10, 40, 10, 50), [(9, 16, 0), (10, 12, 1), (19, 12, 0), (20, 8, 1), (30, 4, 1), (39, 4, 0), (40, 1, 1),
                               (45, 1, 0), (50, 16, 0)]),
    ((8, 4, 0, 7, 4, -1), [(0, 6, 1), (3, 6, 0), (4, 4, 1), (7, 4, 0), (8, 4, 0)]),   # t_end between events
]


@pytest.mark.parametrize("params,table", GMP_HAND)
def test_gmp_schedule_hand_worked(L, params, table):
    for step, n, ev in table:
        flag = ctypes.c_int(7)
        assert L.nm_gmp_n_at(*params, step, ctypes.byref(flag)) == n, (params, step)
        assert flag.value == ev, (params, step)
    assert L.nm_gmp_n_at(8, 8, 0, 4, 1, -1, 0, None) == -1          # n_final must be < M
    assert L.nm_gmp_n_at(8, 2, 5, 4, 1, -1, 0, None) == -1          # t_end < t_begin
    assert L.nm_gmp_n_at(6, 2, 0, 4, 1, -1, 0, None) == -1          # M


def test_mfma_rate_probe_errors(L):
    flops = ctypes.c_int64(0)
    assert L.nm_mfma_rate_probe(0, 16, None, ctypes.byref(flops), None) == nm.NM_ERR_NULL
    assert L.nm_mfma_rate_probe(0, 16, FAKE, None, None) == nm.NM_ERR_NULL
    assert L.nm_mfma_rate_probe(2, 16, FAKE, ctypes.byref(flops), None) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_mfma_rate_probe(1, 0, FAKE, ctypes.byref(flops), None) == nm.NM_ERR_SHAPE
    assert L.nm_mfma_rate_probe(1, 1 << 25, FAKE, ctypes.byref(flops), None) == nm.NM_ERR_SHAPE
    assert L.nm_mfma_rate_probe(0, 16, FAKE + 2, ctypes.byref(flops), None) == nm.NM_ERR_ALIGN
