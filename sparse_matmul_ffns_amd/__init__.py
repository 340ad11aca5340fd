"""MI355X (gfx950) semi-structured sparse FFN matmuls: N:M and V:N:M pruning,
compression and sparse x dense products behind the libnmsparse C ABI.

The binding functions live in `sparse_matmul_ffns_amd.nmsparse`; the library
is loaded on first use and must have been built with
`python -m sparse_matmul_ffns_amd.build`.
"""

from .nmsparse import (  # noqa: F401
    NM_ERR_TOO_LARGE,
    NmError,
    lib,
    mfma_rate_probe,
    nm_compress,
    nm_decompress,
    nm_prune,
    nm_prune_compress,
    nm_prune_compress_transpose,
    nm_reprune_t_transpose,
    nm_reprune_t_transpose_panels,
    nm_to_panels,
    nm_reprune_t,
    prune_act_venom,
    sddmm_nm,
    sizes,
    spmm_nm,
    spmm_nm_general,
    general_work_bytes,
    general_scratch_bytes,
    spmm_nm_general_noalloc,
    sddmm_venom,
    spmm_venom_tn,
    venom_tn_work_bytes,
    spmm_nm_t,
    spmm_nm_t_panels,
    spmm_nm_t_lowrank,
    spmm_nm_t_relu_venom,
    spmm_venom,
    transpose,
)
