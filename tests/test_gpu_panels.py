"""The panel layout on the GPU: nm_to_panels and nm_reprune_t_transpose_panels against the host
reordering of the oracle's row-major forms (byte for byte), spmm_nm_t_panels against spmm_nm_t
(bit for bit: the same products added in the same order) and against the fp64 oracle."""

import numpy as np
import pytest
import torch

import sparse_matmul_ffns_amd as nm
from oracle import nm_oracle as O
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import check_close, dev, host, require_gpu
from tests.panels import meta_to_panels, values_to_panels

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _weight(R, K, seed, kind="normal"):
    raw = synth.small_ints((R, K), seed) if kind == "ints" else synth.normal((R, K), seed, std=0.02)
    vals, meta, _ = O.compress_nm(raw, O.prune_nm(raw, "bf16", 2, 4), 2, 4)
    return raw, vals, meta


@pytest.mark.parametrize("R,K", [(4, 256), (256, 512), (1028, 768)])
def test_to_panels(R, K):
    _, vals, meta = _weight(R, K, R + K)
    vp, mp = nm.nm_to_panels(dev(vals, "bf16"), dev(meta, "u8"), R, K)
    assert host(vp).tobytes() == values_to_panels(vals, R, K).tobytes()
    assert np.array_equal(host(mp), meta_to_panels(meta, R, K))


REPRUNE_CASES = [(256, 128, 72, 136), (512, 384, 1000, 72), (1024, 256, 64, 520)]


@pytest.mark.parametrize("R,K,RX,CX", REPRUNE_CASES, ids=[f"{c[0]}x{c[1]}_X{c[2]}x{c[3]}" for c in REPRUNE_CASES])
def test_reprune_t_transpose_panels(R, K, RX, CX):
    """The re-pruned transpose (K x R, compressed along R) in the panel layout: the oracle's re-prune
    reordered on the host, byte for byte, and nm_to_panels of nm_reprune_t's; Xt exact."""
    _, vals, meta = _weight(R, K, 3 * R + K)
    xraw = synth.normal((RX, CX), RX + CX)
    v, m = dev(vals, "bf16"), dev(meta, "u8")
    vt, mt, Xt = nm.nm_reprune_t_transpose_panels(v, m, R, K, dev(xraw, "bf16"))
    wv, wm = O.reprune_t(vals, meta, R, K, "bf16")
    assert host(vt).tobytes() == values_to_panels(wv, K, R).tobytes()
    assert np.array_equal(host(mt), meta_to_panels(wm, K, R))
    v2, m2 = nm.nm_reprune_t(v, m, R, K)
    p2, q2 = nm.nm_to_panels(v2, m2, K, R)
    assert torch.equal(vt.view(torch.int16), p2.view(torch.int16)) and torch.equal(mt, q2)
    assert np.array_equal(host(Xt), np.ascontiguousarray(xraw.T))


SPMM_CASES = [(256, 256, 256), (512, 768, 264), (256, 1024, 1000), (768, 512, 40), (1024, 2048, 512)]


@pytest.mark.parametrize("R,K,Nc", SPMM_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in SPMM_CASES])
@pytest.mark.parametrize("kind", ["normal", "ints"])
def test_spmm_nm_t_panels(R, K, Nc, kind):
    """Whole and ragged column tiles, one to eight row tiles, K from one 256-column chunk to eight."""
    raw, vals, meta = _weight(R, K, R + 2 * K + Nc, kind)
    Btraw = synth.small_ints((Nc, K), Nc + 1) if kind == "ints" else synth.normal((Nc, K), Nc + 1)
    Bt = dev(Btraw, "bf16")
    vp, mp = dev(values_to_panels(vals, R, K), "bf16"), dev(meta_to_panels(meta, R, K), "u8")
    C = nm.spmm_nm_t_panels(vp, mp, R, K, Bt)
    C_rows = nm.spmm_nm_t(dev(vals, "bf16"), dev(meta, "u8"), K, Bt)
    assert torch.equal(C, C_rows)
    Braw = np.ascontiguousarray(Btraw.T)
    Cref = O.spmm_nm(vals, meta, R, K, Braw, "bf16")
    got = host(C)
    if kind == "ints":
        assert np.array_equal(got, Cref)
    A64 = O.decode(O.decompress_nm(vals, meta, R, K, 2, 4), "bf16")
    check_close(got, Cref, O.abs_bound(A64, O.decode(Braw, "bf16")), f"spmm_nm_t_panels {R}x{K}x{Nc}")


def test_spmm_nm_t_panels_training_step_dx():
    """The training step's input gradient at full size (W_ds^T [4096 x 16384] in the panel layout,
    dY^T [8192 x 16384]): equal to spmm_nm_t bit for bit, twice, and to the oracle on a sampled
    block of 12 rows x 256 columns."""
    R, K, Nc = 4096, 16384, 8192
    g = torch.Generator(device="cuda").manual_seed(5)
    W = (torch.randn(K, R, device="cuda", generator=g) * 0.02).bfloat16()   # W [d_ff x d_model]
    _, v, m = nm.nm_prune_compress(W)
    X = torch.randn(R, 64, device="cuda", generator=g).bfloat16()
    vt, mt, _ = nm.nm_reprune_t_transpose_panels(v, m, K, R, X)
    vr, mr = nm.nm_reprune_t(v, m, K, R)
    dYt = torch.randn(Nc, K, device="cuda", generator=g).bfloat16()
    C = nm.spmm_nm_t_panels(vt, mt, R, K, dYt)
    C2 = nm.spmm_nm_t_panels(vt, mt, R, K, dYt)
    assert torch.equal(C, C2)
    assert torch.equal(C, nm.spmm_nm_t(vr, mr, K, dYt))
    rng = np.random.default_rng(6)
    rows = np.sort(rng.choice(R, 12, replace=False))
    cols = np.sort(rng.choice(Nc, 256, replace=False))
    A64 = O.decode(O.decompress_nm(host(vr)[rows], host(mr)[rows], len(rows), K, 2, 4), "bf16")
    B64 = O.decode(np.ascontiguousarray(host(dYt[torch.as_tensor(cols, device="cuda")]).T), "bf16")
    check_close(host(C)[rows][:, cols], A64 @ B64, O.abs_bound(A64, B64), "spmm_nm_t_panels 4096x16384x8192")
