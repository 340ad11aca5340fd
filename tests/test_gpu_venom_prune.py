"""prune_act_venom (bf16, M = 8, V in {64, 128}) against the fp64 oracle on inputs where the order
of the column additions matters or sits at the edge of mattering.

The rule adds each column's |h| over the V rows in fp64, in row order.  Any other order gives the
same sums only while every addition is exact (the block's nonzero exponents within 45 - log2(V)
of each other).  The order-dependent block below has a column whose row-order sum rounds back to
1.0 at every step while its exact sum exceeds 1.0: only row-order addition keeps the tie (and the
lower column) that the oracle keeps.  Blocks at that exponent bound and one past it, bf16
subnormals, all-zero blocks and grids of many tiles are compared bit for bit as well.
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


def _bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _check(raw, V, relu):
    vals, meta, colsel = nm.prune_act_venom(dev(raw, "bf16"), V, 8, apply_relu=relu)
    wv, wm, wc, _, _ = O.prune_venom(raw, "bf16", V, 8, relu)
    assert np.array_equal(host(colsel), wc)
    assert host(vals).tobytes() == wv.tobytes()
    assert np.array_equal(host(meta), wm)
    return wc


def order_dependent_block(V, K, seed):
    """One V-row block: group 0 holds column 0 = (1.0, 0, ...), column 1 = (1.0, t, t, ...) with t
    below half an ulp of 1.0 (the sequential sum stays 1.0, the exact one does not), columns 2-4
    = 5.0 in row 0; the other groups are N(0, 1)."""
    raw = synth.normal((V, K), seed)
    t = 2.0 ** -58 if V == 64 else 2.0 ** -59
    g0 = np.zeros((V, 8), np.float32)
    g0[0, 0] = g0[0, 1] = 1.0
    g0[1:, 1] = t
    g0[0, 2:5] = 5.0
    raw[:, :8] = _bits(g0)
    return raw


@pytest.mark.parametrize("V", [64, 128])
@pytest.mark.parametrize("relu", [False, True])
def test_order_dependent_column_sums(V, relu):
    K = 512
    raw = np.concatenate([order_dependent_block(V, K, 7), synth.normal((V, K), 8)], axis=0)
    wc = _check(raw, V, relu)
    assert list(wc[0, 0]) == [0, 2, 3, 4]   # the tie of columns 0 and 1 goes to column 0


@pytest.mark.parametrize("V,spread", [(64, 39), (64, 40), (128, 38), (128, 39)])
def test_exponent_spread_at_and_past_the_bound(V, spread):
    """Magnitudes 2^a .. 2^(a + spread) in every tile (random mantissas and signs)."""
    K = 1024
    rng = np.random.Generator(np.random.PCG64(V + spread))
    e = rng.integers(-20, -20 + spread + 1, size=(2 * V, K))
    m = rng.uniform(1.0, 1.99, size=(2 * V, K)) * rng.choice([-1.0, 1.0], size=(2 * V, K))
    raw = _bits(m * np.exp2(e))
    raw[0, ::8] = _bits(np.full(K // 8, 2.0 ** -20))          # the smallest exponent in every tile
    raw[1, ::8] = _bits(np.full(K // 8, 1.5 * 2.0 ** (-20 + spread)))
    _check(raw, V, False)


@pytest.mark.parametrize("V", [64, 128])
def test_subnormals_and_zero_tiles(V):
    K = 768 if V == 64 else 384
    raw = synth.normal((2 * V, K), 11)
    raw[:V, :] = _bits(-np.abs(synth.bf16_bits_to_f32(raw[:V, :])))   # all <= 0: ReLU zeros the block
    sub = np.arange(1, 0x80, dtype=np.uint16)                          # bf16 subnormal bit patterns
    raw[V:, 8:16] = sub[np.arange(V * 8) % len(sub)].reshape(V, 8)
    _check(raw, V, True)
    _check(raw, V, False)


@pytest.mark.parametrize("V,R,K", [(64, 1024, 16384), (128, 1024, 16384), (128, 640, 2176)])
@pytest.mark.parametrize("relu", [False, True])
def test_several_tiles_per_workgroup(V, R, K, relu):
    raw = synth.normal((R, K), R + K, mean=-0.5 if relu else 0.0)
    _check(raw, V, relu)


TILE_CASES = [(V, M, K) for V, K in ((64, 768), (128, 768), (256, 192)) for M in (4, 8, 16)]


@pytest.mark.parametrize("V,M,K", TILE_CASES, ids=[f"V{c[0]}_M{c[1]}_K{c[2]}" for c in TILE_CASES])
@pytest.mark.parametrize("relu", [False, True])
def test_tiled_path_every_v_and_m(V, M, K, relu, monkeypatch):
    """The tiled kernel (bf16, V in {64, 128, 256}, K a multiple of its tile width) for every M, with ties
    in a group of every tile, against the oracle and against the streaming kernel."""
    R = 2 * V
    raw = synth.normal((R, K), V + M + K, mean=-0.5 if relu else 0.0)
    for c in range(0, K, 256 if V == 128 else 16384 // V):
        raw[:V, c:c + M] = synth.tie_rich((V, M), c + 1)
    Z = dev(raw, "bf16")
    vals, meta, colsel = nm.prune_act_venom(Z, V, M, apply_relu=relu)
    wv, wm, wc, _, _ = O.prune_venom(raw, "bf16", V, M, relu)
    assert np.array_equal(host(colsel), wc)
    assert host(vals).tobytes() == wv.tobytes()
    assert np.array_equal(host(meta), wm)
    monkeypatch.setenv("NMSPARSE_VENOM_STREAM", "1")
    sv, sm, sc = nm.prune_act_venom(Z, V, M, apply_relu=relu)
    assert host(sv).tobytes() == host(vals).tobytes()
    assert np.array_equal(host(sm), host(meta)) and np.array_equal(host(sc), host(colsel))
