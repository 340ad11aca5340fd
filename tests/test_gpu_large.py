"""Operands at the size limits of the fast kernels.

Several kernels address an operand with 32-bit byte offsets from a wave-uniform base, and their
dispatch takes them only while that operand is smaller than 4 GiB (2 GiB for the buffer
resource of the register-gather V:N:M SpMM); past the limit the call runs a kernel with 64-bit
addressing.  Each case below is run just under and just over its limit:

  * spmm_nm_t, Bt [Nc][2048] bf16 of 4 GiB - 1 MiB (pipelined kernel) and 4 GiB + 1 MiB (SIMT kernel);
  * spmm_venom (V = 64, M = 8, K = 8192), B [8192][Nc] of 2 GiB - 4 MiB (register-gather kernel)
    and 2 GiB + 4 MiB (direct-to-LDS kernel);
  * sddmm_nm, D [256][T] of 4 GiB - 64 KiB (four-wave kernel) and 4 GiB + 64 KiB (eight-wave kernel).

The large operands are drawn on the device by the counter-based generator of the synthetic inputs
(small integers), and the host regenerates exactly the rows and columns it checks, so every
product is an exact integer: sampled outputs (the first, the last and those around the 2 GiB byte
offset) must equal the fp64 oracle's bit for bit.
"""

import numpy as np
import pytest
import torch

import sparse_matmul_ffns_amd as nm
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _ar(n):
    return torch.arange(n, device="cuda", dtype=torch.int64)


def _samples(n, around):
    s = set(range(4)) | set(range(n - 4, n)) | set(range(around - 4, around + 4))
    return np.array(sorted(x for x in s if 0 <= x < n))


@pytest.mark.parametrize("Nc", [2**20 - 256, 2**20 + 256], ids=["under_4GiB", "over_4GiB"])
def test_spmm_nm_t_bt_at_the_offset_limit(Nc):
    R, K = 256, 2048
    W = synth.small_ints((R, K), 51)
    mask = O.prune_nm(W, "bf16", 2, 4)
    v, m, _ = O.compress_nm(W, mask, 2, 4)
    A64 = O.decode(W, "bf16") * mask
    Bt = synth.hashed_ints_torch(_ar(Nc), _ar(K), 52)          # Bt[n][k]
    C = nm.spmm_nm_t(dev(v, "bf16"), dev(m, "u8"), K, Bt)
    del Bt
    cols = _samples(Nc, 2**31 // (2 * K))                       # the column whose row starts at 2 GiB
    got = host(C[:, torch.as_tensor(cols, device="cuda")]).astype(np.float64)
    ref = A64 @ O.decode(synth.hashed_ints(cols, np.arange(K), 52), "bf16").T
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("Nc", [2**17 - 256, 2**17 + 256], ids=["under_2GiB", "over_2GiB"])
def test_spmm_venom_b_at_the_buffer_limit(Nc):
    R, K, V, M = 128, 8192, 64, 8
    Z = synth.small_ints((R, K), 53)
    vals, meta, colsel, _, _ = O.prune_venom(Z, "bf16", V, M, False)
    A64 = O.decode(O.decompress_venom(vals, meta, colsel, R, K, V, M), "bf16")
    B = synth.hashed_ints_torch(_ar(K), _ar(Nc), 54)            # B[k][n]
    C = nm.spmm_venom(dev(vals, "bf16"), dev(meta, "u8"), dev(colsel, "u8"), K, V, M, B)
    del B
    cols = _samples(Nc, Nc // 2)
    got = host(C[:, torch.as_tensor(cols, device="cuda")]).astype(np.float64)
    ref = A64 @ O.decode(synth.hashed_ints(np.arange(K), cols, 54), "bf16")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("T", [2**23 - 128, 2**23 + 128], ids=["under_4GiB", "over_4GiB"])
def test_sddmm_nm_d_at_the_offset_limit(T):
    R, Kc = 256, 16
    W = synth.small_ints((R, Kc), 55)
    mask = O.prune_nm(W, "bf16", 2, 4)
    _, meta, _ = O.compress_nm(W, mask, 2, 4)
    D = synth.hashed_ints_torch(_ar(R), _ar(T), 56, span=1)     # D[r][t]: |sums| < 2^24, exact
    X = synth.hashed_ints_torch(_ar(Kc), _ar(T), 57, span=1)    # X[c][t]
    dW = nm.sddmm_nm(D, X, dev(meta, "u8"))
    del D, X
    rows = [0, 1, 128, R - 1]
    got = host(dW)[rows].astype(np.float64)
    X64 = O.decode(synth.hashed_ints(np.arange(Kc), np.arange(T), 57, span=1), "bf16")
    for i, r in enumerate(rows):
        D64 = O.decode(synth.hashed_ints([r], np.arange(T), 56, span=1), "bf16")[0]
        kept = np.flatnonzero(mask[r])
        assert np.array_equal(got[i], X64[kept] @ D64), f"row {r}"
