"""Pins of the fp64 oracle to things other than itself (CPU only).

* brute-force enumeration with exact rationals (oracle/brute.py) over
  tie-rich alphabets, exhaustively where the alphabet is small;
* hand-derived examples (tests/golden/hand_examples.json);
* invariants and special cases that reduce to a simpler rule;
* closed forms for the products (an explicit gather loop, exact rational
  products, B = I, linearity).
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import brute
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def f32(a):
    return np.array(a, np.float32)


# ---------------------------------------------------------------------------
# N:M selection against brute force
# ---------------------------------------------------------------------------

ALPHA7 = [-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, 3.0]


@pytest.mark.parametrize("N", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nm_select_exhaustive_m4(N, dtype):
    groups = np.array(list(itertools.product(ALPHA7, repeat=4)), np.float32)  # 2401 groups
    raw = groups if dtype == "f32" else synth.f32_to_bf16_bits(groups)
    got = O.prune_nm(raw, dtype, N, 4)
    want = brute.nm_mask(groups.astype(np.float64), N, 4)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("N", [2, 3])
def test_nm_select_exhaustive_m8(N):
    groups = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=8)), np.float32)  # 6561
    got = O.prune_nm(groups, "f32", N, 8)
    want = brute.nm_mask(groups.astype(np.float64), N, 8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("N,rows", [(2, 40), (4, 20), (8, 2)])
def test_nm_select_random_m16(N, rows):
    raw = synth.tie_rich((rows, 16 * 6), seed=7 + N, dtype="f32")
    got = O.prune_nm(raw, "f32", N, 16)
    want = brute.nm_mask(raw.astype(np.float64), N, 16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# hand-derived examples
# ---------------------------------------------------------------------------

def test_golden_nm24():
    g = GOLDEN["nm24_fp32"]
    A = f32(g["A"])
    mask = O.prune_nm(A, "f32", 2, 4)
    assert mask.tolist() == g["mask"]
    vals, meta, bad = O.compress_nm(A, mask, 2, 4)
    assert bad == 0
    assert vals.tobytes() == f32(g["values"]).tobytes()      # bitwise, signed zeros included
    assert meta.tolist() == g["meta"]
    C = O.spmm_nm(vals, meta, 2, 8, f32(g["B"]), "f32")
    assert C.tolist() == g["C"]


def test_golden_nm28_bit_stream():
    g = GOLDEN["nm28_fp32"]
    A = f32(g["A"])
    mask = O.prune_nm(A, "f32", 2, 8)
    assert mask.tolist() == g["mask"]
    vals, meta, _ = O.compress_nm(A, mask, 2, 8)
    assert vals.tolist() == g["values"]
    assert meta.tolist() == g["meta"]
    back = O.decompress_nm(vals, meta, 1, 16, 2, 8)
    assert np.array_equal(back, np.where(mask == 1, A, 0))


def test_golden_venom():
    g = GOLDEN["vnm_v2_m8_fp32"]
    A = f32(g["A"])
    vals, meta, colsel, mask, _ = O.prune_venom(A, "f32", g["V"], g["M"], apply_relu=False)
    assert colsel.tolist() == g["colsel"]
    assert vals.tolist() == g["values"]
    assert meta.tolist() == g["meta"]
    assert mask.tolist() == g["mask"]


def test_golden_reprune_t():
    g = GOLDEN["reprune_t_fp32"]
    Ws = f32(g["Ws_dense"])
    mask = O.prune_nm(Ws, "f32", 2, 4)
    vals, meta, _ = O.compress_nm(Ws, mask, 2, 4)
    assert vals.tolist() == g["Ws_values"] and meta.tolist() == g["Ws_meta"]
    vt, mt = O.reprune_t(vals, meta, 4, 4, "f32")
    assert vt.tolist() == g["Wt_values"]
    assert mt.tolist() == g["Wt_meta"]


# ---------------------------------------------------------------------------
# invariants of prune + compress
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (2, 8), (4, 8), (4, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prune_compress_invariants(N, M, dtype):
    raw = synth.tie_rich((24, M * 10), seed=N * 100 + M, dtype=dtype)
    raw[:, :M] = synth.normal((24, M), seed=3, dtype=dtype)   # some untied groups too
    x = O.decode(raw, dtype)
    mask = O.prune_nm(raw, dtype, N, M)
    mg = mask.reshape(24, -1, M)
    assert np.all(mg.sum(axis=2) == N)                       # exactly N per group
    keys = np.abs(x).reshape(24, -1, M)
    kept_min = np.where(mg == 1, keys, np.inf).min(axis=2)
    drop_max = np.where(mg == 0, keys, -np.inf).max(axis=2)
    assert np.all(kept_min >= drop_max)                      # kept keys dominate
    vals, meta, bad = O.compress_nm(raw, mask, N, M)
    assert bad == 0
    pos = O.unpack_positions(meta, 24, M * 10, N, M)
    assert np.all(np.diff(pos, axis=2) > 0)                  # ascending positions
    kept_raw = raw.reshape(24, -1, M)[mg == 1].reshape(24, -1)
    assert kept_raw.tobytes() == vals.tobytes()              # raw bits at kept positions
    back = O.decompress_nm(vals, meta, 24, M * 10, N, M)
    want = np.where(mask == 1, raw, O.zeros_raw(raw.shape, dtype))
    assert back.tobytes() == want.tobytes()                  # round trip, +0.0 fill


def test_already_24_is_fixed_point():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((16, 64)).astype(np.float32)
    A = A + np.sign(A) * 0.5                                 # keep away from zero
    sel = O.nm_select(rng.random((16, 64)), 2, 4)            # arbitrary 2:4 pattern
    A = np.where(sel == 1, A, np.float32(0))
    mask = O.prune_nm(A, "f32", 2, 4)
    assert np.array_equal(mask, sel)
    vals, meta, _ = O.compress_nm(A, mask, 2, 4)
    assert O.decompress_nm(vals, meta, 16, 64, 2, 4).tobytes() == A.tobytes()


def test_compress_counts_bad_groups():
    raw = synth.normal((4, 16), seed=1, dtype="bf16")
    mask = O.prune_nm(raw, "bf16", 2, 4)
    mask[0, 0:4] = [1, 1, 1, 0]
    mask[3, 12:16] = [0, 0, 0, 0]
    vals, meta, bad = O.compress_nm(raw, mask, 2, 4)
    assert bad == 2
    assert np.all(vals[0, 0:2] == 0) and np.all(vals[3, 6:8] == 0)
    pos = O.unpack_positions(meta, 4, 16, 2, 4)
    assert pos[0, 0].tolist() == [0, 1] and pos[3, 3].tolist() == [0, 1]


# ---------------------------------------------------------------------------
# V:N:M against brute force and its special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,M", [(1, 8), (2, 8), (3, 8), (2, 16), (4, 4)])
def test_venom_brute(V, M):
    raw = synth.tie_rich((V * 4, M * 5), seed=V * 31 + M, dtype="f32")
    vals, meta, colsel, mask, _ = O.prune_venom(raw, "f32", V, M, apply_relu=False)
    cs, mk = brute.venom_select(raw.astype(np.float64), V, M)
    assert np.array_equal(colsel, cs)
    assert np.array_equal(mask, mk)
    back = O.decompress_venom(vals, meta, colsel, V * 4, M * 5, V, M)
    assert back.tobytes() == np.where(mask == 1, raw, np.float32(0)).tobytes()


def test_venom_m4_is_24():
    raw = synth.normal((32, 64), seed=11, dtype="bf16")
    vals, meta, colsel, mask, _ = O.prune_venom(raw, "bf16", 8, 4, apply_relu=False)
    assert np.all(colsel == np.arange(4))
    m24 = O.prune_nm(raw, "bf16", 2, 4)
    v24, meta24, _ = O.compress_nm(raw, m24, 2, 4)
    assert np.array_equal(mask, m24) and np.array_equal(meta, meta24) and np.array_equal(vals, v24)


def test_venom_v1_is_row_top2_of_8():
    raw = synth.tie_rich((16, 64), seed=12, dtype="bf16")
    _, _, _, mask, _ = O.prune_venom(raw, "bf16", 1, 8, apply_relu=False)
    assert np.array_equal(mask, O.prune_nm(raw, "bf16", 2, 8))


def test_venom_colsel_shared_and_survivors_inside():
    raw = synth.normal((64, 128), seed=13, dtype="bf16")
    V, M = 16, 8
    _, _, colsel, mask, _ = O.prune_venom(raw, "bf16", V, M, apply_relu=False)
    G = 128 // M
    for r in range(64):
        for g in range(G):
            kept = np.nonzero(mask[r, g * M:(g + 1) * M])[0]
            assert len(kept) == 2 and set(kept) <= set(colsel[r // V, g].tolist())
    assert np.all(np.diff(colsel.astype(int), axis=2) > 0)


def test_relu_venom():
    raw = synth.normal((32, 64), seed=14, mean=-0.5, std=1.0, dtype="bf16")
    raw[0, :] = synth.f32_to_bf16_bits(np.full(64, -1.0, np.float32))  # a row with no positives
    raw[1, :8] = synth.f32_to_bf16_bits(np.float32([-0.0] * 8))
    vals, meta, colsel, mask, h = O.prune_venom(raw, "bf16", 8, 8, apply_relu=True)
    hx = O.decode(h, "bf16")
    assert np.all(hx >= 0) and not np.any(np.signbit(hx))   # +0.0 only, no -0.0
    assert np.array_equal(h == 0, ~(O.decode(raw, "bf16") > 0))
    pos = O.unpack_positions(meta, 32, 64 // 8 * 4, 2, 4)
    assert np.all(pos[0] == [0, 1])                          # all-zero row keeps j = 0, 1
    assert np.all(vals[0] == 0)
    cs, mk = brute.venom_select(hx, 8, 8)
    assert np.array_equal(cs, colsel) and np.array_equal(mk, mask)


def test_venom_l1_is_sequential_fp64():
    # Column sums whose fp64 value depends on the order of addition: the rows
    # must be added top to bottom.
    x = np.zeros((4, 8))
    x[:, 0] = [2.0 ** 53, 1.0, 1.0, 0.0]
    l1 = O.venom_column_l1(x, 4, 8)
    assert l1[0, 0] == 2.0 ** 53                              # (2^53 + 1) + 1 rounds twice
    x[:, 0] = [1.0, 1.0, 2.0 ** 53, 0.0]
    assert O.venom_column_l1(x, 4, 8)[0, 0] == 2.0 ** 53 + 2


@pytest.mark.parametrize("V,t", [(64, 2.0 ** -58), (128, 2.0 ** -59)])
def test_venom_sequential_sum_decides_a_tie(V, t):
    """The premise of the GPU test of the order-dependent tile: column 1 = (1, t, t, ...) sums to
    exactly 1.0 in row order (each t is below half an ulp of 1.0), ties column 0 = (1, 0, ...) and
    loses it; its exact sum (what any other order of exact-sum arithmetic would give) exceeds 1.0
    and would win."""
    x = np.zeros((V, 8), np.float32)
    x[0, 0] = x[0, 1] = 1.0
    x[1:, 1] = t
    x[0, 2:5] = 5.0
    raw = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(raw), x)           # every value exact in bf16
    l1 = O.venom_column_l1(O.decode(raw, "bf16"), V, 8)
    assert l1[0, 0] == l1[0, 1] == 1.0
    assert 1.0 + (V - 1) * t > 1.0 + 2.0 ** -53                       # the exact sum rounds up
    _, _, colsel, _, _ = O.prune_venom(raw, "bf16", V, 8, False)
    assert list(colsel[0, 0]) == [0, 2, 3, 4]


# ---------------------------------------------------------------------------
# double pruning
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_reprune_t_brute(seed):
    R, K = 12, 16
    raw = synth.tie_rich((R, K), seed=40 + seed, dtype="f32")
    vals, meta, _ = O.compress_nm(raw, O.prune_nm(raw, "f32", 2, 4), 2, 4)
    vt, mt = O.reprune_t(vals, meta, R, K, "f32")
    ws = np.where(brute.nm_mask(raw.astype(np.float64), 2, 4) == 1, raw, np.float32(0))
    mt_want = brute.nm_mask(ws.T.astype(np.float64), 2, 4)
    back = O.decompress_nm(vt, mt, K, R, 2, 4)
    assert back.tobytes() == np.where(mt_want == 1, ws.T, np.float32(0)).tobytes()


def test_reprune_t_idempotent_on_checkerboard():
    # 2x2 blocks in a checkerboard are 2:4 along rows and along columns.
    i, j = np.indices((16, 16))
    pat = (((i // 2) + (j // 2)) % 2 == 0).astype(np.float64)
    rng = np.random.default_rng(3)
    mag = rng.integers(1, 9, pat.shape) * rng.choice([-1, 1], pat.shape)
    A = np.where(pat == 1, mag, 0.0).astype(np.float32)        # +0.0 off the pattern
    vals, meta, _ = O.compress_nm(A, O.prune_nm(A, "f32", 2, 4), 2, 4)
    assert O.decompress_nm(vals, meta, 16, 16, 2, 4).tobytes() == A.tobytes()
    vt, mt = O.reprune_t(vals, meta, 16, 16, "f32")
    assert O.decompress_nm(vt, mt, 16, 16, 2, 4).tobytes() == np.ascontiguousarray(A.T).tobytes()


# ---------------------------------------------------------------------------
# products: closed forms
# ---------------------------------------------------------------------------

def _compressed(R, K, seed, dtype, ints=False):
    raw = synth.small_ints((R, K), seed, dtype=dtype) if ints else synth.normal((R, K), seed, dtype=dtype)
    vals, meta, _ = O.compress_nm(raw, O.prune_nm(raw, dtype, 2, 4), 2, 4)
    return raw, vals, meta


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_spmm_gather_loop_equals_dgemm(dtype):
    R, K, Nc = 6, 24, 5
    _, vals, meta = _compressed(R, K, 50, dtype)
    B = synth.normal((K, Nc), 51, dtype=dtype)
    a = O.spmm_nm(vals, meta, R, K, B, dtype)
    b = O.spmm_nm_loop(vals, meta, R, K, B, dtype)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_spmm_exact_rational():
    R, K, Nc = 5, 16, 4
    _, vals, meta = _compressed(R, K, 52, "f32")
    B = synth.normal((K, Nc), 53, dtype="f32")
    A64 = O.decode(O.decompress_nm(vals, meta, R, K, 2, 4), "f32")
    exact = brute.dense_product(A64, B.astype(np.float64))
    assert np.allclose(O.spmm_nm(vals, meta, R, K, B, "f32"), exact, rtol=1e-14, atol=1e-14)


def test_spmm_identity_and_linearity():
    R, K = 8, 32
    raw, vals, meta = _compressed(R, K, 54, "bf16", ints=True)
    eye = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    C = O.spmm_nm(vals, meta, R, K, eye, "bf16")
    assert np.array_equal(C, O.decode(O.decompress_nm(vals, meta, R, K, 2, 4), "bf16"))
    B1 = synth.small_ints((K, 3), 55, dtype="bf16")
    B2 = synth.small_ints((K, 3), 56, dtype="bf16")
    Bs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(B1) + synth.bf16_bits_to_f32(B2))
    assert np.array_equal(O.spmm_nm(vals, meta, R, K, Bs, "bf16"),
                          O.spmm_nm(vals, meta, R, K, B1, "bf16") + O.spmm_nm(vals, meta, R, K, B2, "bf16"))


@pytest.mark.parametrize("N,M", [(1, 4), (2, 8), (4, 8), (3, 8), (4, 16)])
def test_spmm_general_gather_loop_and_exact_integers(N, M):
    R, K, Nc = 5, 4 * M, 4
    raw = synth.small_ints((R, K), 90 + N + M, dtype="bf16")
    vals, meta, _ = O.compress_nm(raw, O.prune_nm(raw, "bf16", N, M), N, M)
    B = synth.small_ints((K, Nc), 91 + N + M, dtype="bf16")
    C = O.spmm_nm_general(vals, meta, R, K, N, M, B, "bf16")
    assert np.array_equal(C, O.spmm_nm_general_loop(vals, meta, R, K, N, M, B, "bf16"))
    # exact integer sums over the kept positions, straight from the mask
    mask = O.prune_nm(raw, "bf16", N, M)
    a = synth.bf16_bits_to_f32(raw).astype(np.int64) * mask
    b = synth.bf16_bits_to_f32(B).astype(np.int64)
    assert np.array_equal(C, (a @ b).astype(np.float64))


def test_spmm_general_2of4_is_spmm_nm():
    R, K = 6, 32
    _, vals, meta = _compressed(R, K, 95, "bf16")
    B = synth.normal((K, 3), 96, dtype="bf16")
    assert np.array_equal(O.spmm_nm_general(vals, meta, R, K, 2, 4, B, "bf16"), O.spmm_nm(vals, meta, R, K, B, "bf16"))


def test_spmm_venom_gather_loop_equals_dgemm():
    R, K, V, M, Nc = 8, 32, 4, 8, 5
    raw = synth.normal((R, K), 60, dtype="bf16")
    vals, meta, colsel, _, _ = O.prune_venom(raw, "bf16", V, M, apply_relu=False)
    B = synth.normal((K, Nc), 61, dtype="bf16")
    a = O.spmm_venom(vals, meta, colsel, R, K, V, M, B, "bf16")
    b = O.spmm_venom_loop(vals, meta, colsel, R, K, V, M, B, "bf16")
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# backward of the V:N:M down-projection: loop forms, adjoint identities with the
# forward SpMM, the M = 4 case, the ReLU gate
# ---------------------------------------------------------------------------

def _venom_bwd_case(T, F, Nc, V, M, seed, ints, relu=True):
    gen = synth.small_ints if ints else synth.normal
    z = gen((T, F), seed, dtype="bf16")
    hv, hm, hc, _, _ = O.prune_venom(z, "bf16", V, M, apply_relu=relu)
    dY = gen((T, Nc), seed + 1, dtype="bf16")
    Wd = gen((F, Nc), seed + 2, dtype="bf16")
    return hv, hm, hc, dY, Wd


@pytest.mark.parametrize("relu", [False, True])
def test_sddmm_venom_loop_and_exact_integers(relu):
    T, F, Nc, V, M = 8, 32, 5, 4, 8
    for ints in (False, True):
        hv, hm, hc, dY, Wd = _venom_bwd_case(T, F, Nc, V, M, 80 + ints, ints, relu)
        a = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu)
        b = O.sddmm_venom_loop(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu)
        assert np.array_equal(a, b) if ints else np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_spmm_venom_tn_loop_and_exact_integers():
    T, F, Nc, V, M = 8, 48, 6, 2, 16
    for ints in (False, True):
        hv, hm, hc, dY, _ = _venom_bwd_case(T, F, Nc, V, M, 84 + ints, ints)
        a = O.spmm_venom_tn(hv, hm, hc, T, F, V, M, dY, "bf16")
        b = O.spmm_venom_tn_loop(hv, hm, hc, T, F, V, M, dY, "bf16")
        assert np.array_equal(a, b) if ints else np.allclose(a, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("V,M", [(4, 8), (2, 4), (8, 16), (1, 8)])
def test_venom_backward_adjoint_identities(V, M):
    """<h_s W, dY> = <h_s^T dY, W> = sum over kept entries of h * (dY W^T): the two backward
    products are the adjoints of the pinned forward product (exact on integers)."""
    T, F, Nc = 16, 4 * M, 6
    hv, hm, hc, dY, Wd = _venom_bwd_case(T, F, Nc, V, M, 90 + M, True, relu=False)
    Y = O.spmm_venom(hv, hm, hc, T, F, V, M, Wd, "bf16")
    dW = O.spmm_venom_tn(hv, hm, hc, T, F, V, M, dY, "bf16")
    dz = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu=False)
    lhs = float(np.sum(Y * O.decode(dY, "bf16")))
    assert lhs == float(np.sum(dW * O.decode(Wd, "bf16")))
    assert lhs == float(np.sum(O.decode(hv, "bf16") * dz))


def test_sddmm_venom_m4_is_sddmm_nm():
    """M = 4 keeps every column (colsel = 0..3), so the V:N:M SDDMM is the 2:4 SDDMM with h_s's
    nibbles."""
    T, F, Nc, V = 8, 16, 7, 4
    hv, hm, hc, dY, Wd = _venom_bwd_case(T, F, Nc, V, 4, 95, False, relu=False)
    assert (hc == np.arange(4, dtype=np.uint8)).all()
    assert np.array_equal(O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, 4, "bf16", relu=False),
                          O.sddmm_nm(dY, Wd, hm, T, F, "bf16"))


def test_sddmm_venom_relu_gate():
    T, F, Nc, V, M = 8, 32, 4, 4, 8
    hv, hm, hc, dY, Wd = _venom_bwd_case(T, F, Nc, V, M, 97, False, relu=True)
    gated = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu=True)
    plain = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu=False)
    pos = O.decode(hv, "bf16") > 0
    assert 0 < pos.sum() < pos.size                     # both kinds of kept entries occur
    assert np.array_equal(gated[pos], plain[pos]) and not gated[~pos].any()


def test_gmp_schedule_hand_worked():
    """The oracle's schedule against the hand-worked tables (the rule stated in its comment)."""
    from tests.test_abi import GMP_HAND
    for params, table in GMP_HAND:
        for step, n, ev in table:
            assert O.gmp_n_at(*params, step) == (n, bool(ev)), (params, step)


def test_gmp_schedule_properties():
    for M, nf in [(4, 2), (4, 1), (8, 2), (8, 6), (16, 1)]:
        for begin, end, interval in [(0, 0, 1), (3, 20, 4), (5, 50, 7)]:
            ns = [O.gmp_n_at(M, nf, begin, end, interval, end + 10, t)[0] for t in range(end + 12)]
            sparse = ns[begin:end + 10]
            assert all(a >= b for a, b in zip(sparse, sparse[1:]))          # monotone ramp
            assert sparse[-1] == nf and max(sparse) < M                     # reaches the target; every event prunes
            assert ns[:begin] == [M] * begin and ns[end + 10:] == [M] * 2   # dense before and after


def test_abs_bound_hand_values():
    # |A| |B| by hand: [[1*1 + 2*2, 1*4 + 2*5], [0*1 + 3*2, 0*4 + 3*5]]
    A = np.array([[1.0, -2.0], [0.0, 3.0]])
    B = np.array([[-1.0, 4.0], [2.0, -5.0]])
    assert np.array_equal(O.abs_bound(A, B), np.array([[5.0, 14.0], [6.0, 15.0]]))
    # a product that cancels to zero keeps its full bound
    assert np.array_equal(O.abs_bound(np.array([[1.0, 1.0]]), np.array([[1.0], [-1.0]])), np.array([[2.0]]))


def test_sddmm_exact_rational():
    R, Kc, T = 4, 8, 6
    D = synth.small_ints((R, T), 70, dtype="bf16")
    X = synth.small_ints((Kc, T), 71, dtype="bf16")
    W = synth.normal((R, Kc), 72, dtype="bf16")
    _, meta, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    got = O.sddmm_nm(D, X, meta, R, Kc, "bf16")
    full = brute.dense_product(O.decode(D, "bf16"), O.decode(X, "bf16").T)
    pos = O.unpack_positions(meta, R, Kc, 2, 4)
    for r in range(R):
        for g in range(Kc // 4):
            for s in range(2):
                assert got[r, 2 * g + s] == full[r, 4 * g + pos[r, g, s]]
    rows = np.array([3, 1])
    assert np.array_equal(O.sddmm_nm_rows(D, X, meta, rows, Kc, "bf16"), got[rows])


# ---------------------------------------------------------------------------
# sparse plus low-rank: exact integer sums, the adapted weight, special cases
# ---------------------------------------------------------------------------

def _lowrank_case(R, K, Nc, r, seed, ints):
    gen = synth.small_ints if ints else synth.normal
    raw, vals, meta = _compressed(R, K, seed, "bf16", ints=ints)
    B = gen((K, Nc), seed + 1, dtype="bf16")
    U = gen((R, r), seed + 2, dtype="bf16")
    Vt = gen((r, K), seed + 3, dtype="bf16")
    return raw, vals, meta, B, U, Vt


def test_spmm_lowrank_exact_integers():
    # small integers: every sum is an integer far below 2**53, so the float64 result must equal
    # the integer arithmetic done here element by element
    R, K, Nc, r = 6, 16, 5, 3
    raw, vals, meta, B, U, Vt = _lowrank_case(R, K, Nc, r, 80, ints=True)
    C, T = O.spmm_nm_lowrank(vals, meta, R, K, B, U, Vt, "bf16")
    mask = O.prune_nm(raw, "bf16", 2, 4)
    a = [[int(v) for v in row] for row in synth.bf16_bits_to_f32(raw)]
    b = [[int(v) for v in row] for row in synth.bf16_bits_to_f32(B)]
    u = [[int(v) for v in row] for row in synth.bf16_bits_to_f32(U)]
    vt = [[int(v) for v in row] for row in synth.bf16_bits_to_f32(Vt)]
    for j in range(r):
        for n in range(Nc):
            assert T[j, n] == sum(vt[j][k] * b[k][n] for k in range(K))
    for i in range(R):
        for n in range(Nc):
            sparse = sum(a[i][k] * b[k][n] for k in range(K) if mask[i, k])
            adapter = sum(u[i][j] * sum(vt[j][k] * b[k][n] for k in range(K)) for j in range(r))
            assert C[i, n] == sparse + adapter


def test_spmm_lowrank_is_the_adapted_weight_times_b():
    # (W_s + U Vt) B, formed densely, is the same product evaluated in another order
    R, K, Nc, r = 12, 32, 7, 4
    _, vals, meta, B, U, Vt = _lowrank_case(R, K, Nc, r, 84, ints=False)
    C, _ = O.spmm_nm_lowrank(vals, meta, R, K, B, U, Vt, "bf16")
    W = O.decode(O.decompress_nm(vals, meta, R, K, 2, 4), "bf16") + O.decode(U, "bf16") @ O.decode(Vt, "bf16")
    assert np.allclose(C, W @ O.decode(B, "bf16"), rtol=1e-12, atol=1e-12)


def test_spmm_lowrank_special_cases():
    R, K, Nc, r = 8, 16, 6, 2
    _, vals, meta, B, U, Vt = _lowrank_case(R, K, Nc, r, 88, ints=True)
    zeroU = np.zeros_like(U)
    C, T = O.spmm_nm_lowrank(vals, meta, R, K, B, zeroU, Vt, "bf16")
    assert np.array_equal(C, O.spmm_nm(vals, meta, R, K, B, "bf16"))
    # one-hot factors: the adapter adds row k = 5 of B to output row i = 3 (and nothing else)
    one = synth.f32_to_bf16_bits(np.float32([1.0]))[0]
    Ue = np.zeros_like(U)
    Ue[3, 1] = one
    Ve = np.zeros_like(Vt)
    Ve[1, 5] = one
    C, T = O.spmm_nm_lowrank(vals, meta, R, K, B, Ue, Ve, "bf16")
    want = O.spmm_nm(vals, meta, R, K, B, "bf16")
    want[3] += O.decode(B, "bf16")[5]
    assert np.array_equal(C, want)
    assert np.array_equal(T[1], O.decode(B, "bf16")[5]) and not T[0].any()
    rows = np.array([6, 0, 3])
    assert np.array_equal(O.spmm_nm_lowrank_rows(vals, meta, rows, K, B, Ue, Ve, "bf16"), C[rows])


def test_tolerance_check():
    ref = np.array([[1.0, -2.0]])
    bound = np.array([[1.0, 2.0]])
    assert O.within_tolerance(ref + 1e-4, ref, bound)[0]
    assert not O.within_tolerance(ref + np.array([[0.0, 0.05]]), ref, bound)[0]


def test_decode_bf16():
    bits = np.array([0x3F80, 0xBF80, 0x8000, 0x0000, 0x4049, 0x0001], np.uint16)
    got = O.decode(bits, "bf16")
    assert got[:4].tolist() == [1.0, -1.0, 0.0, 0.0] and np.signbit(got[2])
    assert got[4] == 3.140625 and got[5] == 2.0 ** -133


# ---------------------------------------------------------------------------
# encode_bf16: float64 -> nearest bf16, ties to even (products stored in bf16)
# ---------------------------------------------------------------------------

def test_encode_bf16_known_values():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -2.5, 0.0, -0.0,
                  (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40), 3.4e38,
                  2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 - 2.0 ** -134])
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000,
            0x7F7F, 0x7F7F, 0x7F80,
            0x0001, 0x0000, 0x0001, 0x0080]
    assert O.encode_bf16(x).tolist() == want


def test_encode_bf16_round_trips_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    assert np.array_equal(O.encode_bf16(O.decode(bits[finite], "bf16")), bits[finite])


def test_encode_bf16_is_nearest_ties_even_brute():
    """Against the two neighbouring bf16 values found by search over all patterns."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 127, 3000))
    x = np.concatenate([x, (O.decode(np.arange(0x0001, 0x7F7F, 97, dtype=np.uint16), "bf16")
                            + O.decode(np.arange(0x0002, 0x7F80, 97, dtype=np.uint16), "bf16")) / 2])  # exact ties
    pos = np.sort(O.decode(np.arange(0x0000, 0x7F80, dtype=np.uint16), "bf16"))   # all finite bf16 >= 0
    got = O.decode(O.encode_bf16(x), "bf16")
    for xi, gi in zip(x, got):
        a = abs(xi)
        i = np.searchsorted(pos, a, side="right") - 1          # pos[i] <= a < pos[i+1]
        lo, hi = pos[i], (pos[i + 1] if i + 1 < len(pos) else np.inf)
        if a - lo < hi - a:
            want = lo
        elif a - lo > hi - a:
            want = hi
        else:                                                 # tie: the even pattern
            want = lo if (i % 2 == 0) else hi
        assert abs(gi) == want and (gi == 0 or np.sign(gi) == np.sign(xi)), (xi, gi, want)


def test_encode_bf16_matches_fp32_bit_rounding():
    """For fp32 inputs, the same result as rounding the fp32 bit pattern (add 0x7FFF plus the
    lowest kept bit, drop the low 16 bits)."""
    rng = np.random.default_rng(6)
    u = rng.integers(0, 0x7F7F0000, 20000, dtype=np.uint64).astype(np.uint32)
    u |= (rng.integers(0, 2, 20000).astype(np.uint32) << np.uint32(31))
    f = u.view(np.float32)
    want = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(O.encode_bf16(f.astype(np.float64)), want)

