"""spmm_nm_general_noalloc (the general N:M SpMM with the library's fixed scratch buffer instead
of caller work memory) against spmm_nm_general with work memory: the same kernels, so the same
bits, and both within the fp64 oracle's tolerance.  Two calls in a row on one GPU, the second
with a smaller input (the buffer keeps the first call's bytes beyond the second's rewrite), then
a pattern with dense rows in the buffer, one that needs no scratch at all, and an fp32 call.
"""

import numpy as np
import pytest
import torch

import sparse_matmul_ffns_amd as nm
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import check_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(R, K, N, M, Nc, seed, dtype="bf16", kind="normal"):
    W = synth.normal((R, K), seed, std=0.02, dtype=dtype) if kind == "normal" else \
        synth.small_ints((R, K), seed, dtype=dtype)
    vals, meta, _ = O.compress_nm(W, O.prune_nm(W, dtype, N, M), N, M)
    Bt = synth.normal((Nc, K), seed + 1, dtype=dtype) if kind == "normal" else \
        synth.small_ints((Nc, K), seed + 1, dtype=dtype)
    v, m, b = dev(vals, dtype), dev(meta, "u8"), dev(Bt, dtype)
    out = torch.full((R, Nc), float("nan"), device="cuda")
    nm.spmm_nm_general_noalloc(v, m, K, N, M, b, out)
    want = nm.spmm_nm_general(v, m, K, N, M, b)          # the existing entry point, work memory from torch
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"{N}:{M} {R}x{K}x{Nc}"
    ref = O.spmm_nm_general(vals, meta, R, K, N, M, np.ascontiguousarray(Bt.T), dtype)
    if kind == "ints":
        assert np.array_equal(host(out), ref)
    A64 = O.decode(O.decompress_nm(vals, meta, R, K, N, M), dtype)
    check_close(host(out), ref, O.abs_bound(A64, O.decode(np.ascontiguousarray(Bt.T), dtype)),
                f"noalloc {N}:{M} {R}x{K}x{Nc}")


def test_noalloc_two_calls_second_smaller():
    assert nm.general_scratch_bytes() == 64 << 20
    assert nm.general_work_bytes(torch.bfloat16, 2048, 4096, 2, 8) <= nm.general_scratch_bytes()
    _run(2048, 4096, 2, 8, 520, 31)               # 2:8: rewritten into the scratch buffer (18.9 MB)
    _run(256, 512, 1, 4, 264, 32)                 # smaller, 1:4: the start of the buffer again
    _run(512, 1024, 2, 16, 136, 33, kind="ints")  # bit-exact integers
    _run(256, 512, 4, 8, 72, 34)                  # 4:8: dense bf16 rows in the scratch buffer
    _run(64, 96, 3, 4, 40, 36)                    # 3:4 with K % 64 != 0: no scratch (SIMT kernel)
    _run(128, 256, 2, 8, 64, 35, dtype="f32")     # fp32 2:8 through the scratch buffer


def test_noalloc_rejects_too_large():
    R, K = 65536, 1024
    v = torch.zeros((R, K // 8 * 2), dtype=torch.bfloat16, device="cuda")
    m = torch.zeros((R, nm.sizes(R, K, 2, 8)[1] // R), dtype=torch.uint8, device="cuda")
    b = torch.zeros((8, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((R, 8), 7.0, device="cuda")
    with pytest.raises(nm.NmError) as e:
        nm.spmm_nm_general_noalloc(v, m, K, 2, 8, b, out)
    assert e.value.status == nm.NM_ERR_TOO_LARGE
    assert bool((out == 7.0).all())
