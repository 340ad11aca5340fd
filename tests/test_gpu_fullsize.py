"""GPU parity at the full sizes of the four FFN workloads, through the same
entry points, shapes and seeds the benchmark times (so the same kernel
instantiations and launch grids run).

Selection results (masks, compressed values, metadata, column selections,
re-pruned transposes) are compared bit for bit with the fp64 oracle over the
whole matrix (the [8192 x 16384] activation prune included: the oracle prunes
it once and the forward and backward tests share the result).  Matmul outputs are checked on
sampled rows (and, where the oracle's dense operand fits, sampled columns):
the oracle computes those outputs one by one in fp64 from its own compressed
operands and the seeded inputs, and the acceptance test is the usual one
(relative Frobenius <= 1e-3 and |C - C*| <= 1e-2 (|A| |B|) elementwise).
Every output of the GPU must also be finite.
"""

import numpy as np
import pytest
import torch

import sparse_matmul_ffns_amd as nm
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import check_close, dev, host, require_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gen(spec, shape):
    return synth.normal(shape, spec["seed"], spec["mean"], spec["std"], "bf16")


def _sample(n_total, n, seed, tile=256):
    """Sorted sample of indices: random ones plus the first and last index and
    both sides of the first tile boundary."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(n_total, size=min(n, n_total), replace=False).tolist())
    pick |= {0, n_total - 1, min(tile - 1, n_total - 1), min(tile, n_total - 1)}
    return np.array(sorted(pick), dtype=np.int64)


def _finite(t: torch.Tensor, what: str):
    assert bool(torch.isfinite(t).all()), f"{what}: non-finite output"


def _check_rows(C_dev, A64_rows, B64, rows, what):
    """C[rows, :] against A64_rows @ B64 (A64_rows are the oracle's dense rows)."""
    got = host(C_dev[torch.as_tensor(rows, device=C_dev.device)])
    check_close(got, A64_rows @ B64, O.abs_bound(A64_rows, B64), f"{what} rows")


def _check_cols(C_dev, A64, B64_cols, cols, what):
    got = host(C_dev[:, torch.as_tensor(cols, device=C_dev.device)])
    check_close(got, A64 @ B64_cols, O.abs_bound(A64, B64_cols), f"{what} columns")


# ---------------------------------------------------------------------------
# 2:4 up-projection: nm_prune -> nm_compress -> spmm_nm (and nm_transpose -> spmm_nm_t),
# W [8192 x 2048], X [2048 x 4096]
# ---------------------------------------------------------------------------

def test_ffn_up_nm24_full():
    w = synth.WORKLOADS["ffn_up_nm24_8192x2048x4096"]
    R, K, Nc = w["R"], w["K"], w["Nc"]
    W, X = _gen(w["A"], (R, K)), _gen(w["B"], (K, Nc))
    Wd, Xd = dev(W, "bf16"), dev(X, "bf16")

    mask = nm.nm_prune(Wd)
    want_mask = O.prune_nm(W, "bf16", 2, 4)
    assert np.array_equal(host(mask), want_mask)
    vals, meta = nm.nm_compress(Wd, mask)
    wv, wm, bad = O.compress_nm(W, want_mask, 2, 4)
    assert bad == 0
    assert host(vals).tobytes() == wv.tobytes()
    assert np.array_equal(host(meta), wm)

    C = nm.spmm_nm(vals, meta, K, Xd)
    _finite(C, "spmm_nm")
    A64 = O.decode(O.decompress_nm(wv, wm, R, K, 2, 4), "bf16")
    X64 = O.decode(X, "bf16")
    rows = _sample(R, 48, 11)
    _check_rows(C, A64[rows], X64, rows, "ffn_up spmm_nm")
    cols = _sample(Nc, 24, 12)
    _check_cols(C, A64, X64[:, cols], cols, "ffn_up spmm_nm")
    del C

    # the same product from the K-contiguous activations: nm_transpose, then spmm_nm_t
    Xt = nm.transpose(Xd)
    assert np.array_equal(host(Xt[:64]), np.ascontiguousarray(X[:, :64].T))
    C = nm.spmm_nm_t(vals, meta, K, Xt)
    _finite(C, "spmm_nm_t")
    _check_rows(C, A64[rows], X64, rows, "ffn_up spmm_nm_t")
    _check_cols(C, A64, X64[:, cols], cols, "ffn_up spmm_nm_t")
    del C, Xt

    # the benchmark's step: nm_prune_compress_transpose (one launch), then spmm_nm_t
    fmask, fvals, fmeta, fXt = nm.nm_prune_compress_transpose(Wd, Xd)
    assert np.array_equal(host(fmask), want_mask)
    assert host(fvals).tobytes() == wv.tobytes()
    assert np.array_equal(host(fmeta), wm)
    assert np.array_equal(host(fXt), np.ascontiguousarray(X.T))
    C = nm.spmm_nm_t(fvals, fmeta, K, fXt)
    _finite(C, "spmm_nm_t after nm_prune_compress_transpose")
    _check_rows(C, A64[rows], X64, rows, "ffn_up fused prep + spmm_nm_t")


# ---------------------------------------------------------------------------
# 2:4 up-projection with a rank-64 adapter: nm_prune_compress_transpose -> spmm_nm_t_lowrank,
# W [8192 x 2048], X [2048 x 4096], U [8192 x 64], Vt [64 x 2048]
# ---------------------------------------------------------------------------

def test_ffn_up_nm24_lowrank64_full():
    w = synth.WORKLOADS["ffn_up_nm24_lowrank64_8192x2048x4096"]
    R, K, Nc, r = w["R"], w["K"], w["Nc"], w["rank"]
    W, X = _gen(w["A"], (R, K)), _gen(w["B"], (K, Nc))
    U, Vt = _gen(w["U"], (R, r)), _gen(w["Vt"], (r, K))
    _, fvals, fmeta, fXt = nm.nm_prune_compress_transpose(dev(W, "bf16"), dev(X, "bf16"))
    C, Tt = nm.spmm_nm_t_lowrank(fvals, fmeta, K, fXt, dev(U, "bf16"), dev(Vt, "bf16"))
    _finite(C, "spmm_nm_t_lowrank")
    wv, wm, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    assert host(fvals).tobytes() == wv.tobytes() and np.array_equal(host(fmeta), wm)
    X64, U64, Vt64 = O.decode(X, "bf16"), O.decode(U, "bf16"), O.decode(Vt, "bf16")
    T64 = Vt64 @ X64                                           # [r, Nc], the oracle's inner activations
    Tbound = O.abs_bound(Vt64, X64)
    check_close(host(Tt), T64.T, Tbound.T, "lowrank Tt")
    rows = _sample(R, 48, 13)
    want = O.spmm_nm_lowrank_rows(wv, wm, rows, K, X, U, Vt, "bf16")
    A64r = O.decode(O.decompress_nm(wv[rows], wm[rows], len(rows), K, 2, 4), "bf16")
    bound = O.abs_bound(A64r, X64) + O.abs_bound(U64[rows], Tbound)
    got = host(C[torch.as_tensor(rows, device=C.device)])
    check_close(got, want, bound, "ffn_up lowrank rows")


# ---------------------------------------------------------------------------
# 2:8 and 4:8 up-projections: nm_prune_compress_transpose (N:M) -> spmm_nm_general (2:8: the 2:4
# form in work memory; 4:8: dense bf16 rows in work memory and the dense GEMM),
# W [8192 x 2048], X [2048 x 4096]
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["ffn_up_nm28_8192x2048x4096", "ffn_up_nm48_8192x2048x4096"])
def test_ffn_up_general_full(name):
    w = synth.WORKLOADS[name]
    R, K, Nc, N, M = w["R"], w["K"], w["Nc"], w["N"], w["M"]
    W, X = _gen(w["A"], (R, K)), _gen(w["B"], (K, Nc))
    fmask, fvals, fmeta, fXt = nm.nm_prune_compress_transpose(dev(W, "bf16"), dev(X, "bf16"), N, M)
    want_mask = O.prune_nm(W, "bf16", N, M)
    assert np.array_equal(host(fmask), want_mask)
    wv, wm, _ = O.compress_nm(W, want_mask, N, M)
    assert host(fvals).tobytes() == wv.tobytes() and np.array_equal(host(fmeta), wm)
    work = torch.empty(nm.general_work_bytes(torch.bfloat16, R, K, N, M), dtype=torch.uint8, device="cuda")
    C = nm.spmm_nm_general(fvals, fmeta, K, N, M, fXt, work=work)
    _finite(C, "spmm_nm_general")
    A64 = O.decode(O.decompress_nm(wv, wm, R, K, N, M), "bf16")
    X64 = O.decode(X, "bf16")
    rows = _sample(R, 48, 17)
    _check_rows(C, A64[rows], X64, rows, f"ffn_up {N}:{M} spmm_nm_general")
    cols = _sample(Nc, 24, 18)
    _check_cols(C, A64, X64[:, cols], cols, f"ffn_up {N}:{M} spmm_nm_general")


# ---------------------------------------------------------------------------
# V:N:M (V=64, M=8) down-projection: prune_act_venom -> spmm_venom,
# W [2048 x 8192], X [8192 x 4096]
# ---------------------------------------------------------------------------

def test_ffn_down_vnm64_full():
    w = synth.WORKLOADS["ffn_down_vnm64_2_8_2048x8192x4096"]
    R, K, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
    W, X = _gen(w["A"], (R, K)), _gen(w["B"], (K, Nc))
    Wd, Xd = dev(W, "bf16"), dev(X, "bf16")

    vals, meta, colsel = nm.prune_act_venom(Wd, V, M, apply_relu=False)
    wv, wm, wc, _, _ = O.prune_venom(W, "bf16", V, M, False)
    assert np.array_equal(host(colsel), wc)
    assert host(vals).tobytes() == wv.tobytes()
    assert np.array_equal(host(meta), wm)

    C = nm.spmm_venom(vals, meta, colsel, K, V, M, Xd)
    _finite(C, "spmm_venom")
    A64 = O.decode(O.decompress_venom(wv, wm, wc, R, K, V, M), "bf16")
    X64 = O.decode(X, "bf16")
    rows = _sample(R, 48, 21, tile=V)
    _check_rows(C, A64[rows], X64, rows, "ffn_down spmm_venom")
    cols = _sample(Nc, 24, 22)
    _check_cols(C, A64, X64[:, cols], cols, "ffn_down spmm_venom")


# ---------------------------------------------------------------------------
# ReLU activations pruned V:N:M (V=128, M=8) per step, then h_s @ W_down:
# Z [8192 x 16384], W_down [16384 x 4096]
# ---------------------------------------------------------------------------

_ORACLE_CACHE = {}


def _oracle_relu_prune(w):
    """The oracle's ReLU + V:N:M prune of the workload's whole activation matrix (computed once)."""
    key = (w["Z"]["seed"], w["R"], w["K"], w["V"], w["M"])
    if key not in _ORACLE_CACHE:
        Z = _gen(w["Z"], (w["R"], w["K"]))
        wv, wm, wc, _, _ = O.prune_venom(Z, "bf16", w["V"], w["M"], True)
        _ORACLE_CACHE[key] = (Z, wv, wm, wc)
    return _ORACLE_CACHE[key]


def test_relu_act_vnm128_full():
    """The activation prune over the whole [8192 x 16384] matrix, bit for bit (all 64 V-blocks);
    the down-projection on sampled rows of sampled blocks."""
    w = synth.WORKLOADS["relu_act_vnm128_2_8_8192x16384x4096"]
    R, K, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
    Z, wv, wm, wc = _oracle_relu_prune(w)
    Wdn = _gen(w["W"], (K, Nc))
    Zd, Wdd = dev(Z, "bf16"), dev(Wdn, "bf16")

    vals, meta, colsel = nm.prune_act_venom(Zd, V, M, apply_relu=True)
    C = nm.spmm_venom(vals, meta, colsel, K, V, M, Wdd)
    _finite(C, "spmm_venom")
    assert np.array_equal(host(colsel), wc), "colsel"
    assert host(vals).tobytes() == wv.tobytes(), "values"
    assert np.array_equal(host(meta), wm), "metadata"
    del vals, meta, colsel, Zd

    rng = np.random.default_rng(31)
    W64 = O.decode(Wdn, "bf16")
    for b in sorted({0, R // V - 1} | set(rng.choice(R // V, 4, replace=False).tolist())):
        rs = slice(b * V, (b + 1) * V)
        A64 = O.decode(O.decompress_venom(wv[rs], wm[rs], wc[b:b + 1], V, K, V, M), "bf16")
        rows = np.array(sorted({0, V - 1} | set(rng.choice(V, 6, replace=False).tolist())))
        _check_rows(C, A64[rows], W64, b * V + rows, f"relu_act block {b} spmm_venom")


def test_relu_act_vnm128_bwd_full():
    """The backward of the same down-projection at full size, from the oracle's own activations
    (bit-identical to the GPU's, above): dZ on sampled tokens, dY^T over the whole matrix, dW_down
    on sampled rows (every column)."""
    w = synth.WORKLOADS["relu_act_vnm128_bwd_8192x16384x4096"]
    T, F, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
    Z, wv, wm, wc = _oracle_relu_prune(w)
    Wd = _gen(w["W"], (F, Nc))
    dY = _gen(w["dY"], (T, Nc))
    hv, hm, hc = nm.prune_act_venom(dev(Z, "bf16"), V, M, apply_relu=True)
    assert host(hv).tobytes() == wv.tobytes() and np.array_equal(host(hm), wm) and np.array_equal(host(hc), wc)
    dYd = dev(dY, "bf16")
    dz, dYt = nm.sddmm_venom(dYd, dev(Wd, "bf16"), hv, hm, hc, V, M, apply_relu=True,
                             dYt=torch.empty((Nc, T), dtype=torch.bfloat16, device="cuda"))
    dW = nm.spmm_venom_tn(hv, hm, hc, F, V, M, dYt)
    _finite(dz, "sddmm_venom")
    _finite(dW, "spmm_venom_tn")
    assert np.array_equal(host(dYt), np.ascontiguousarray(dY.T)), "dY^T"
    del hv, hm, hc, dYd

    # dZ on sampled tokens: the oracle's SDDMM restricted to those rows (rows are independent)
    toks = _sample(T, 24, 41, tile=128)
    got = host(dz[torch.as_tensor(toks, device="cuda")])
    ref = O.sddmm_venom(dY[toks], Wd, wv[toks], wm[toks], wc[toks // V], len(toks), F, 1, M, "bf16", True)
    full = np.abs(O.decode(dY[toks], "bf16")) @ np.abs(O.decode(Wd, "bf16")).T
    bound = np.take_along_axis(full, O.venom_kept_columns(wm[toks], wc[toks // V], len(toks), F, 1, M), axis=1)
    check_close(got, ref, bound, "sddmm_venom sampled tokens")

    # dW_down on sampled rows k: sum over every token of h_s[t][k] dY[t]
    ks = _sample(F, 24, 42)
    Hraw = O.decompress_venom(wv, wm, wc, T, F, V, M)
    Hk = O.decode(np.ascontiguousarray(Hraw[:, ks]), "bf16")            # [T, len(ks)]
    del Hraw
    dY64 = O.decode(dY, "bf16")
    got = host(dW[torch.as_tensor(ks, device="cuda")])
    check_close(got, Hk.T @ dY64, O.abs_bound(np.abs(Hk.T), dY64), "spmm_venom_tn sampled rows")


# ---------------------------------------------------------------------------
# the FFN block forward: 2:4 up-projection (bf16 output) -> token-major h -> ReLU + V:N:M (V=128,
# M=8) -> V:N:M down-projection; d_model 4096, d_ff 16384, 8192 tokens
# ---------------------------------------------------------------------------

def test_ffn_block_fwd_full():
    """Small-integer inputs, so that every up-projection sum is an exact fp32 integer and its bf16
    rounding is the oracle's: the V:N:M selection of the activations is then compared bit for bit
    on sampled V-blocks, and the down-projection on sampled tokens within tolerance."""
    w = synth.WORKLOADS["ffn_block_fwd_nm24_vnm128_dmodel4096_dff16384_tok8192"]
    dm, dff, T, V, M = w["d_model"], w["d_ff"], w["tokens"], w["V"], w["M"]
    W = synth.small_ints((dff, dm), 71, dtype="bf16")
    Xt = synth.small_ints((T, dm), 72, dtype="bf16")
    Wd = synth.small_ints((dff, dm), 73, dtype="bf16")
    _, vals, meta = nm.nm_prune_compress(dev(W, "bf16"))
    hT = nm.spmm_nm_t(vals, meta, dm, dev(Xt, "bf16"), out_dtype=torch.bfloat16)
    h = nm.transpose(hT)
    del hT
    hv, hm, hc = nm.prune_act_venom(h, V, M, apply_relu=True)
    del h
    Y = nm.spmm_venom(hv, hm, hc, dff, V, M, dev(Wd, "bf16"))
    _finite(Y, "ffn block")
    # the fused up-projection (ReLU + V:N:M in its epilogue) gives the same compressed activations
    fv, fm, fc = nm.spmm_nm_t_relu_venom(vals, meta, dm, dev(Xt, "bf16"), V, M)
    assert torch.equal(fc, hc) and torch.equal(fv.view(torch.int16), hv.view(torch.int16)) and torch.equal(fm, hm)
    del fv, fm, fc
    gv, gm, gc = host(hv), host(hm), host(hc)
    wv, wm, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    assert host(vals).tobytes() == wv.tobytes() and np.array_equal(host(meta), wm)
    Ws64 = O.decode(O.decompress_nm(wv, wm, dff, dm, 2, 4), "bf16")
    Wd64 = O.decode(Wd, "bf16")
    rng = np.random.default_rng(74)
    for b in sorted({0, T // V - 1} | set(rng.choice(T // V, 1, replace=False).tolist())):
        ts = slice(b * V, (b + 1) * V)
        Z = O.decode(Xt[ts], "bf16") @ Ws64.T                      # exact integers, [V, d_ff]
        ov, om, oc, _, _ = O.prune_venom(O.encode_bf16(Z), "bf16", V, M, True)
        assert np.array_equal(gc[b:b + 1], oc), f"colsel of block {b}"
        assert gv[ts].tobytes() == ov.tobytes(), f"values of block {b}"
        assert np.array_equal(gm[ts], om), f"metadata of block {b}"
        H64 = O.decode(O.decompress_venom(ov, om, oc, V, dff, V, M), "bf16")
        rows = np.array(sorted({0, V - 1} | set(rng.choice(V, 4, replace=False).tolist())))
        _check_rows(Y, H64[rows], Wd64, b * V + rows, f"ffn block {b} down-projection")


# ---------------------------------------------------------------------------
# 2:4 double-pruned training step: d_model 4096, d_ff 16384, 8192 tokens
#   Y = W_s X, W_ds^T = re-prune(W_s^T), dX = W_ds^T dY, dW = (dY X^T) at W_s's pattern
# ---------------------------------------------------------------------------

def test_train_step_nm24_full():
    w = synth.WORKLOADS["train_step_nm24_dmodel4096_dff16384_tok8192"]
    dm, dff, T = w["d_model"], w["d_ff"], w["tokens"]
    W = _gen(w["W"], (dff, dm))
    X = _gen(w["X"], (dm, T))
    dY = _gen(w["dY"], (dff, T))
    Wd, Xd, dYd = dev(W, "bf16"), dev(X, "bf16"), dev(dY, "bf16")

    mask = nm.nm_prune(Wd)
    want_mask = O.prune_nm(W, "bf16", 2, 4)
    assert np.array_equal(host(mask), want_mask)
    vals, meta = nm.nm_compress(Wd, mask)
    wv, wm, bad = O.compress_nm(W, want_mask, 2, 4)
    assert bad == 0
    assert host(vals).tobytes() == wv.tobytes() and np.array_equal(host(meta), wm)
    del mask, want_mask, Wd

    # the step's first launch: W_ds^T and X^T together; then the re-prune alone, which must agree
    vt, mt, Xt = nm.nm_reprune_t_transpose(vals, meta, dff, dm, Xd)
    wvt, wmt = O.reprune_t(wv, wm, dff, dm, "bf16")
    assert host(vt).tobytes() == wvt.tobytes()
    assert np.array_equal(host(mt), wmt)
    assert np.array_equal(host(Xt), np.ascontiguousarray(X.T))
    vt2, mt2 = nm.nm_reprune_t(vals, meta, dff, dm)
    assert torch.equal(vt2.view(torch.int16), vt.view(torch.int16)) and torch.equal(mt2, mt)
    del vt2, mt2

    X64 = O.decode(X, "bf16")
    # forward: Y = W_s X
    Y = nm.spmm_nm(vals, meta, dm, Xd)
    _finite(Y, "Y")
    rows = _sample(dff, 32, 41)
    Ws_rows = O.decode(O.decompress_nm(wv[rows], wm[rows], len(rows), dm, 2, 4), "bf16")
    _check_rows(Y, Ws_rows, X64, rows, "train Y")
    del Y
    Y = nm.spmm_nm_t(vals, meta, dm, Xt)
    del Xt
    _finite(Y, "Y (spmm_nm_t)")
    _check_rows(Y, Ws_rows, X64, rows, "train Y (spmm_nm_t)")
    del Y

    # dX = W_ds^T dY
    dX = nm.spmm_nm(vt, mt, dff, dYd)
    _finite(dX, "dX")
    rows = _sample(dm, 24, 42)
    Wt_rows = O.decode(O.decompress_nm(wvt[rows], wmt[rows], len(rows), dff, 2, 4), "bf16")
    _check_rows(dX, Wt_rows, O.decode(dY, "bf16"), rows, "train dX")
    del dX
    dX = nm.spmm_nm_t(vt, mt, dff, nm.transpose(dYd))
    _finite(dX, "dX (spmm_nm_t)")
    _check_rows(dX, Wt_rows, O.decode(dY, "bf16"), rows, "train dX (spmm_nm_t)")
    del dX

    # dW = (dY X^T) read at W_s's kept positions
    dW = nm.sddmm_nm(dYd, Xd, meta)
    _finite(dW, "dW")
    rows = _sample(dff, 32, 43)
    ref = O.sddmm_nm_rows(dY, X, wm, rows, dm, "bf16")
    D64 = O.decode(dY[rows], "bf16")
    full_bound = np.abs(D64) @ np.abs(X64).T
    pos = O.unpack_positions(wm[rows], len(rows), dm, 2, 4)
    cols = (np.arange(dm // 4)[None, :, None] * 4 + pos).reshape(len(rows), dm // 2)
    got = host(dW[torch.as_tensor(rows, device=dW.device)])
    check_close(got, ref, np.take_along_axis(full_bound, cols, axis=1), "train dW rows")
    del dW

    # the benchmark's order: dW with sddmm_nm_dt (which also writes dY^T), then dX from that dY^T
    dW, dYt = nm.sddmm_nm(dYd, Xd, meta, Dt=torch.empty((T, dff), dtype=torch.bfloat16, device="cuda"))
    got = host(dW[torch.as_tensor(rows, device=dW.device)])
    check_close(got, ref, np.take_along_axis(full_bound, cols, axis=1), "train dW rows (sddmm_nm_dt)")
    del dW
    assert np.array_equal(host(dYt), np.ascontiguousarray(dY.T))
    dX = nm.spmm_nm_t(vt, mt, dff, dYt)
    _finite(dX, "dX after sddmm_nm_dt")
    xrows = _sample(dm, 24, 42)   # the rows Wt_rows holds
    _check_rows(dX, Wt_rows, O.decode(dY, "bf16"), xrows, "train dX from sddmm_nm_dt's dY^T")
