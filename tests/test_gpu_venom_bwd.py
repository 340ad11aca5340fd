"""GPU parity of the V:N:M down-projection's backward (sddmm_venom, spmm_venom_tn) against the
fp64 oracle: bit-exact on small integers (every partial sum exact in fp32), within the stated
tolerance otherwise; the matrix-core tiers and the SIMT tiers; ragged shapes; run-twice identity.
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


def _case(T, F, Nc, V, M, seed, kind, dtype="bf16", relu=True):
    gen = synth.small_ints if kind == "ints" else synth.normal
    z = gen((T, F), seed, dtype=dtype) if kind == "ints" else synth.normal((T, F), seed, mean=-0.5, dtype=dtype)
    hv, hm, hc, _, _ = O.prune_venom(z, dtype, V, M, apply_relu=relu)
    dY = gen((T, Nc), seed + 1, dtype=dtype)
    Wd = gen((F, Nc), seed + 2, dtype=dtype) if kind == "ints" else synth.normal((F, Nc), seed + 2, std=0.02,
                                                                                   dtype=dtype)
    return hv, hm, hc, dY, Wd


def _dz_bound(dY, Wd, hm, hc, T, F, V, M, dtype):
    full = np.abs(O.decode(dY, dtype)) @ np.abs(O.decode(Wd, dtype)).T
    return np.take_along_axis(full, O.venom_kept_columns(hm, hc, T, F, V, M), axis=1)


SDDMM_VENOM_CASES = [
    # (T, F, Nc, V, M): V % 128 == 0 and Nc % 64 == 0 take the matrix-core kernel
    (256, 512, 128, 128, 8),      # one 512-wide gathered tile, only 256 columns of it in range
    (384, 2048, 256, 128, 8),     # three V-blocks, two column tiles, four stages
    (256, 1024, 384, 256, 16),    # M = 16, six stages
    (256, 256, 256, 128, 4),      # M = 4, four stages
    (384, 2048, 192, 128, 8),     # three V-blocks, two column tiles, three 64-wide stages
    (256, 256, 64, 128, 4),       # M = 4: colsel 0..3
    (256, 1024, 128, 256, 16),    # M = 16, a 256-token V-block over two row tiles
    (192, 512, 128, 64, 8),       # V = 64: SIMT kernel
    (128, 256, 72, 128, 8),       # Nc % 64 != 0: SIMT kernel
]


@pytest.mark.parametrize("T,F,Nc,V,M", SDDMM_VENOM_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}_V{c[3]}_M{c[4]}"
                                                              for c in SDDMM_VENOM_CASES])
@pytest.mark.parametrize("kind", ["normal", "ints"])
@pytest.mark.parametrize("relu", [True, False])
@pytest.mark.parametrize("with_dt", [True, False])
def test_sddmm_venom(T, F, Nc, V, M, kind, relu, with_dt):
    hv, hm, hc, dY, Wd = _case(T, F, Nc, V, M, T + F + Nc + M, kind, relu=relu)
    dt_buf = torch.full((Nc, T + 8), 3, dtype=torch.int16, device="cuda").view(torch.bfloat16) if with_dt else None
    res = nm.sddmm_venom(dev(dY, "bf16"), dev(Wd, "bf16"), dev(hv, "bf16"), dev(hm, "u8"), dev(hc, "u8"), V, M,
                         apply_relu=relu, dYt=dt_buf[:, :T] if with_dt else None)
    dz = host(res[0] if with_dt else res)
    ref = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "bf16", relu)
    if kind == "ints":
        assert np.array_equal(dz, ref)
    check_close(dz, ref, _dz_bound(dY, Wd, hm, hc, T, F, V, M, "bf16"), f"sddmm_venom {T}x{F}x{Nc}")
    if with_dt:
        assert np.array_equal(host(res[1]), np.ascontiguousarray(dY.T))
        assert bool((dt_buf.view(torch.int16)[:, T:] == 3).all())


def test_sddmm_venom_fp32():
    T, F, Nc, V, M = 64, 128, 40, 16, 8
    hv, hm, hc, dY, Wd = _case(T, F, Nc, V, M, 7, "normal", dtype="f32")
    dz = host(nm.sddmm_venom(dev(dY, "f32"), dev(Wd, "f32"), dev(hv, "f32"), dev(hm, "u8"), dev(hc, "u8"), V, M))
    ref = O.sddmm_venom(dY, Wd, hv, hm, hc, T, F, V, M, "f32", True)
    check_close(dz, ref, _dz_bound(dY, Wd, hm, hc, T, F, V, M, "f32"), "sddmm_venom fp32")


TN_CASES = [
    # (T, F, Nc, V, M, pad_out): bf16 with work, T % 64 == 0 and ldo % 4 == 0 take the expansion + NT GEMM
    (256, 512, 256, 128, 8, 0),
    (512, 1024, 320, 64, 8, 0),    # ragged column tile
    (192, 256, 70, 64, 4, 2),      # 70 columns in rows of 72: the last four-column piece is partial
    (128, 768, 128, 32, 16, 0),
    (100, 96, 24, 4, 8, 0),        # T % 64 != 0: SIMT kernel
]


@pytest.mark.parametrize("T,F,Nc,V,M,pad", TN_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}_V{c[3]}_M{c[4]}" for c in TN_CASES])
@pytest.mark.parametrize("kind", ["normal", "ints"])
@pytest.mark.parametrize("work", ["auto", None])
def test_spmm_venom_tn(T, F, Nc, V, M, pad, kind, work):
    hv, hm, hc, dY, _ = _case(T, F, Nc, V, M, 3 * T + F + Nc, kind)
    dYt = dev(np.ascontiguousarray(dY.T), "bf16")
    big = torch.full((F + 1, Nc + pad), float("nan"), device="cuda")
    out = big[:F, :Nc]
    nm.spmm_venom_tn(dev(hv, "bf16"), dev(hm, "u8"), dev(hc, "u8"), F, V, M, dYt, out=out, work=work)
    dW = host(out.contiguous())
    ref = O.spmm_venom_tn(hv, hm, hc, T, F, V, M, dY, "bf16")
    if kind == "ints":
        assert np.array_equal(dW, ref)
    H = O.decode(O.decompress_venom(hv, hm, hc, T, F, V, M), "bf16")
    check_close(dW, ref, O.abs_bound(np.abs(H.T), O.decode(dY, "bf16")), f"spmm_venom_tn {T}x{F}x{Nc}")
    assert torch.isnan(big[:F, Nc:]).all() and torch.isnan(big[F:]).all()


def test_spmm_venom_tn_fp32():
    T, F, Nc, V, M = 64, 64, 24, 8, 8
    hv, hm, hc, dY, _ = _case(T, F, Nc, V, M, 11, "normal", dtype="f32")
    dW = host(nm.spmm_venom_tn(dev(hv, "f32"), dev(hm, "u8"), dev(hc, "u8"), F, V, M,
                               dev(np.ascontiguousarray(dY.T), "f32")))
    ref = O.spmm_venom_tn(hv, hm, hc, T, F, V, M, dY, "f32")
    H = O.decode(O.decompress_venom(hv, hm, hc, T, F, V, M), "f32")
    check_close(dW, ref, O.abs_bound(np.abs(H.T), O.decode(dY, "f32")), "spmm_venom_tn fp32")


def test_venom_backward_twice_and_tiers_agree(monkeypatch):
    """Both calls are deterministic, and the SIMT tier reproduces the matrix-core tier within the
    tolerance (exactly on integers)."""
    T, F, Nc, V, M = 512, 1024, 256, 128, 8
    hv, hm, hc, dY, Wd = _case(T, F, Nc, V, M, 21, "ints")
    args = (dev(dY, "bf16"), dev(Wd, "bf16"), dev(hv, "bf16"), dev(hm, "u8"), dev(hc, "u8"), V, M)
    a, b = nm.sddmm_venom(*args), nm.sddmm_venom(*args)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    dYt = dev(np.ascontiguousarray(dY.T), "bf16")
    w1 = nm.spmm_venom_tn(args[2], args[3], args[4], F, V, M, dYt)
    w2 = nm.spmm_venom_tn(args[2], args[3], args[4], F, V, M, dYt)
    assert torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    monkeypatch.setenv("NMSPARSE_FORCE_GENERIC", "1")
    assert torch.equal(nm.sddmm_venom(*args), a)
    assert torch.equal(nm.spmm_venom_tn(args[2], args[3], args[4], F, V, M, dYt), w1)


def test_venom_backward_rejects():
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8, device="cuda")
    with pytest.raises(nm.NmError):   # T % V != 0
        nm.sddmm_venom(z(100, 64), z(64, 64), z(100, 16), u8(100, 4), u8(1, 8, 4), 128, 8)
    with pytest.raises(nm.NmError):   # M = 5
        nm.spmm_venom_tn(z(128, 16), u8(128, 4), u8(1, 8, 4), 40, 128, 5, z(8, 128))


@pytest.mark.parametrize("T,F,Nc,V,M", [(256, 512, 256, 128, 8), (192, 256, 72, 64, 4), (128, 1024, 64, 64, 16),
                                        (512, 384, 136, 256, 8)])
def test_spmm_venom_tn_expansions_agree(T, F, Nc, V, M, monkeypatch):
    """The vector expansion of h_s^T and the scattering one (NMSPARSE_EXPAND_SCATTER=1) give the same
    dW_down bit for bit, for every M; both against the oracle on small integers (exact)."""
    hv, hm, hc, dY, _ = _case(T, F, Nc, V, M, 5 * T + F, "ints")
    args = (dev(hv, "bf16"), dev(hm, "u8"), dev(hc, "u8"), F, V, M, dev(np.ascontiguousarray(dY.T), "bf16"))
    a = nm.spmm_venom_tn(*args, work="auto")
    monkeypatch.setenv("NMSPARSE_EXPAND_SCATTER", "1")
    b = nm.spmm_venom_tn(*args, work="auto")
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert np.array_equal(host(a), O.spmm_venom_tn(hv, hm, hc, T, F, V, M, dY, "bf16"))
