"""Degenerate shapes: one row, one column, one group, one V-block of one row.

Every entry point at the smallest shapes its definition allows (a single 2:4 group, a single
output row or column, V = 1, R = 4 for the transposed re-prune), with bf16 and fp32, against the
fp64 oracle.  Inputs are small integers with ties, so products are exact and every output is
compared bit for bit.
"""

import numpy as np
import pytest

import sparse_matmul_ffns_amd as nm
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ints(shape, seed, dt):
    return synth.small_ints(shape, seed, lo=-2, hi=2, dtype="bf16" if dt == "bf16" else "f32")


SHAPES = [(1, 4, 1), (1, 256, 8), (4, 4, 1), (3, 16, 3), (1, 8, 300)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("R,K,Nc", SHAPES)
def test_prune_compress_spmm_tiny(R, K, Nc, dt):
    A = _ints((R, K), R * 100 + K, dt)
    B = _ints((K, Nc), K + Nc, dt)
    mask = O.prune_nm(A, dt, 2, 4)
    v, m, _ = O.compress_nm(A, mask, 2, 4)
    gmask, gv, gm = nm.nm_prune_compress(dev(A, dt))
    assert np.array_equal(host(gmask), mask)
    assert host(gv).tobytes() == v.tobytes() and np.array_equal(host(gm), m)
    ref = O.spmm_nm(v, m, R, K, B, dt)
    assert np.array_equal(host(nm.spmm_nm(gv, gm, K, dev(B, dt))).astype(np.float64), ref)
    Bt = np.ascontiguousarray(B.T)
    assert np.array_equal(host(nm.spmm_nm_t(gv, gm, K, dev(Bt, dt))).astype(np.float64), ref)


@pytest.mark.parametrize("R,Kc,T", [(1, 4, 1), (1, 8, 3), (5, 4, 2), (2, 4, 130)])
def test_sddmm_tiny(R, Kc, T):
    W = _ints((R, Kc), 7 + R, "bf16")
    _, meta, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    D, X = _ints((R, T), 8 + T, "bf16"), _ints((Kc, T), 9 + T, "bf16")
    got = host(nm.sddmm_nm(dev(D, "bf16"), dev(X, "bf16"), dev(meta, "u8")))
    assert np.array_equal(got.astype(np.float64), O.sddmm_nm(D, X, meta, R, Kc, "bf16"))


@pytest.mark.parametrize("V,M,R,K,Nc", [(1, 4, 1, 4, 1), (1, 8, 3, 8, 5), (2, 4, 2, 4, 7), (4, 16, 4, 16, 2)])
@pytest.mark.parametrize("relu", [False, True])
def test_venom_tiny(V, M, R, K, Nc, relu):
    Z = _ints((R, K), V + M + R + K, "bf16")
    B = _ints((K, Nc), 11 + Nc, "bf16")
    wv, wm, wc, _, _ = O.prune_venom(Z, "bf16", V, M, relu)
    vals, meta, colsel = nm.prune_act_venom(dev(Z, "bf16"), V, M, apply_relu=relu)
    assert host(vals).tobytes() == wv.tobytes()
    assert np.array_equal(host(meta), wm) and np.array_equal(host(colsel), wc)
    C = host(nm.spmm_venom(vals, meta, colsel, K, V, M, dev(B, "bf16")))
    assert np.array_equal(C.astype(np.float64), O.spmm_venom(wv, wm, wc, R, K, V, M, B, "bf16"))


@pytest.mark.parametrize("R,K", [(4, 4), (4, 8), (8, 4)])
def test_reprune_t_tiny(R, K):
    W = _ints((R, K), 13 + R + K, "bf16")
    v, m, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    wvt, wmt = O.reprune_t(v, m, R, K, "bf16")
    gvt, gmt = nm.nm_reprune_t(dev(v, "bf16"), dev(m, "u8"), R, K)
    assert host(gvt).tobytes() == wvt.tobytes() and np.array_equal(host(gmt), wmt)
