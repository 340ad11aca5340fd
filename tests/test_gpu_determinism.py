"""Run-twice bit identity and guard canaries for the kernels of the path.

Every call is deterministic: the same inputs give the same bytes on a second
call (each kernel sums in a fixed order; no atomics).  Outputs that are views
into larger buffers must leave everything outside the view untouched: the
surrounding memory is filled with a sentinel pattern and compared afterwards.
Shapes span several tiles and end in partial tiles; the ragged SDDMM case is the
one whose last row panel has waves with no rows in range.
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


def _same(a, b):
    """Bitwise equality of tensors (or tuples of tensors): NaN patterns and signed zeros count."""
    if isinstance(a, (tuple, list)):
        return len(a) == len(b) and all(_same(x, y) for x, y in zip(a, b))
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16}.get(a.dtype)
    return torch.equal(a.view(view), b.view(view)) if view else torch.equal(a, b)


def _bf16(shape, seed, std=1.0, mean=0.0):
    return dev(synth.normal(shape, seed, std=std, mean=mean), "bf16")


@pytest.mark.parametrize("tier", ["reg", "dma"])
@pytest.mark.parametrize("R,K,Nc,V", [(1024, 2048, 1032, 64), (1024, 4096, 768, 128)])
def test_spmm_venom_twice(R, K, Nc, V, tier, monkeypatch):
    if tier == "dma":
        monkeypatch.setenv("NMSPARSE_SPMM_TIER", "2")
    v, m, c = nm.prune_act_venom(_bf16((R, K), 1, 0.02), V, 8)
    B = _bf16((K, Nc), 2)
    assert _same(nm.spmm_venom(v, m, c, K, V, 8, B), nm.spmm_venom(v, m, c, K, V, 8, B))


@pytest.mark.parametrize("R,Kc,T", [(300, 520, 256), (512, 1024, 512), (1000, 264, 192)])
def test_sddmm_dt_twice_and_oracle(R, Kc, T):
    """sddmm_nm_dt twice (bit-identical dW and dY^T) and against the oracle, including partial last
    row panels (R % 256 in 1..192, where some waves of the panel have no rows)."""
    Draw = synth.normal((R, T), 5, dtype="bf16")
    Xraw = synth.normal((Kc, T), 6, dtype="bf16")
    W = synth.normal((R, Kc), 7, dtype="bf16")
    vals, meta, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    D, X, mt = dev(Draw, "bf16"), dev(Xraw, "bf16"), dev(meta, "u8")
    out1, dt1 = nm.sddmm_nm(D, X, mt, Dt=torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
    out2, dt2 = nm.sddmm_nm(D, X, mt, Dt=torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
    assert _same(out1, out2) and _same(dt1, dt2)
    assert np.array_equal(host(dt1), np.ascontiguousarray(Draw.T))
    ref = O.sddmm_nm(Draw, Xraw, meta, R, Kc, "bf16")
    full_bound = np.abs(O.decode(Draw, "bf16")) @ np.abs(O.decode(Xraw, "bf16")).T
    pos = O.unpack_positions(meta, R, Kc, 2, 4)
    cols = (np.arange(Kc // 4)[None, :, None] * 4 + pos).reshape(R, Kc // 2)
    check_close(host(out1), ref, np.take_along_axis(full_bound, cols, axis=1), f"sddmm_nm_dt {R}x{Kc}x{T}")


@pytest.mark.parametrize("relu", [False, True])
def test_prune_act_venom_twice(relu):
    Z = _bf16((512, 4096), 8, 1.0, -0.5)
    assert _same(nm.prune_act_venom(Z, 128, 8, apply_relu=relu), nm.prune_act_venom(Z, 128, 8, apply_relu=relu))


def test_spmm_nm_t_relu_venom_twice():
    R, K, Nc = 512, 1024, 512
    v, m = nm.nm_prune_compress(_bf16((R, K), 9, 0.02))[1:]
    Bt = _bf16((Nc, K), 10)
    assert _same(nm.spmm_nm_t_relu_venom(v, m, K, Bt), nm.spmm_nm_t_relu_venom(v, m, K, Bt))


def test_reprune_and_spmm_t_twice():
    R, K, Nc = 1024, 768, 520
    v, m = nm.nm_prune_compress(_bf16((R, K), 11, 0.02))[1:]
    assert _same(nm.nm_reprune_t(v, m, R, K), nm.nm_reprune_t(v, m, R, K))
    Bt = _bf16((Nc, K), 12)
    assert _same(nm.spmm_nm_t(v, m, K, Bt), nm.spmm_nm_t(v, m, K, Bt))


SENTINEL = float("nan")


@pytest.mark.parametrize("tier", ["reg", "dma"])
def test_spmm_venom_guard(tier, monkeypatch):
    """C written through a strided view: padding columns and the rows after it keep the sentinel."""
    if tier == "dma":
        monkeypatch.setenv("NMSPARSE_SPMM_TIER", "2")
    R, K, Nc, V = 512, 1024, 264, 64
    v, m, c = nm.prune_act_venom(_bf16((R, K), 13, 0.02), V, 8)
    B = _bf16((K, Nc), 14)
    big = torch.full((R + 3, Nc + 24), SENTINEL, device="cuda")
    nm.spmm_venom(v, m, c, K, V, 8, B, out=big[:R, :Nc])
    want = nm.spmm_venom(v, m, c, K, V, 8, B)
    assert _same(big[:R, :Nc].contiguous(), want)
    assert torch.isnan(big[:R, Nc:]).all() and torch.isnan(big[R:]).all()


def test_spmm_nm_t_guard():
    R, K, Nc = 520, 512, 264
    v, m = nm.nm_prune_compress(_bf16((R, K), 15, 0.02))[1:]
    Bt = _bf16((Nc, K), 16)
    big = torch.full((R + 2, Nc + 8), SENTINEL, device="cuda")
    nm.spmm_nm_t(v, m, K, Bt, out=big[:R, :Nc])
    assert _same(big[:R, :Nc].contiguous(), nm.spmm_nm_t(v, m, K, Bt))
    assert torch.isnan(big[:R, Nc:]).all() and torch.isnan(big[R:]).all()


def test_sddmm_guard():
    """dW into the head of a larger flat buffer and dY^T into a strided view: the rest keeps the
    sentinel (the partial last row panel has waves with no rows in range)."""
    R, Kc, T = 300, 264, 128
    D, X = _bf16((R, T), 17), _bf16((Kc, T), 18)
    W = synth.normal((R, Kc), 19, dtype="bf16")
    _, meta, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
    mt = dev(meta, "u8")
    flat = torch.full((R * (Kc // 2) + 64,), SENTINEL, device="cuda")
    dtbig = torch.full((T, R + 8), -1.0, device="cuda").to(torch.bfloat16)
    out, dt = nm.sddmm_nm(D, X, mt, out=flat[:R * (Kc // 2)].view(R, Kc // 2), Dt=dtbig[:, :R])
    ref_out, ref_dt = nm.sddmm_nm(D, X, mt, Dt=torch.empty((T, R), dtype=torch.bfloat16, device="cuda"))
    assert _same(out.contiguous(), ref_out) and _same(dt.contiguous(), ref_dt)
    assert torch.isnan(flat[R * (Kc // 2):]).all()
    assert (dtbig[:, R:].float() == -1.0).all()
