"""The hot path's steps captured into a HIP graph and replayed.

No call of the library allocates device memory, clears memory or synchronises, so a whole step
(several calls on one stream, outputs allocated beforehand) can be recorded once and replayed:
the form a serving or training loop uses to drop the host's per-launch cost.  Each step is run
eagerly first; then it is captured, and every one of three replays, with eager work of the
program's own (clearing the outputs) and a synchronisation between them, must reproduce the eager
outputs bit for bit.
"""

import pytest
import torch

import sparse_matmul_ffns_amd as nm
from sparse_matmul_ffns_amd import synth
from tests.gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _up24():
    """2:4 up-projection: one-launch prune + compress + transpose, then the K-contiguous SpMM."""
    R, K, Nc = 512, 512, 768
    W, X = dev(synth.normal((R, K), 1, std=0.02), "bf16"), dev(synth.normal((K, Nc), 2), "bf16")
    mask = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    vals = torch.empty((R, K // 2), dtype=torch.bfloat16, device="cuda")
    meta = torch.empty((R, K // 8), dtype=torch.uint8, device="cuda")
    Bt = torch.empty((Nc, K), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")

    def step():
        nm.nm_prune_compress_transpose(W, X, mask=mask, values=vals, meta=meta, Bt=Bt)
        nm.spmm_nm_t(vals, meta, K, Bt, out=C)
    return step, [mask, vals, meta, Bt, C]


def _train():
    """Double-pruned training step: re-pruned transpose in the panel layout with X's transpose, Y,
    dW with dY^T, dX on the panel layout."""
    dff, dm, T = 512, 512, 384
    W = synth.normal((dff, dm), 3, std=0.02)
    X, dY = dev(synth.normal((dm, T), 4), "bf16"), dev(synth.normal((dff, T), 5), "bf16")
    vals, meta = nm.nm_compress(dev(W, "bf16"), nm.nm_prune(dev(W, "bf16")))
    vt = torch.empty((dm * dff // 2,), dtype=torch.bfloat16, device="cuda")
    mt = torch.empty((dm * dff // 8,), dtype=torch.uint8, device="cuda")
    Xt = torch.empty((T, dm), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((dff, T), dtype=torch.float32, device="cuda")
    dW = torch.empty((dff, dm // 2), dtype=torch.float32, device="cuda")
    dYt = torch.empty((T, dff), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((dm, T), dtype=torch.float32, device="cuda")

    def step():
        nm.nm_reprune_t_transpose_panels(vals, meta, dff, dm, X, values_t=vt, meta_t=mt, Xt=Xt)
        nm.spmm_nm_t(vals, meta, dm, Xt, out=Y)
        nm.sddmm_nm(dY, X, meta, out=dW, Dt=dYt)
        nm.spmm_nm_t_panels(vt, mt, dm, dff, dYt, out=dX)
    return step, [vt, mt, Xt, Y, dW, dYt, dX]


def _vnm():
    """ReLU + V:N:M activation prune (V = 64, M = 8), then the V:N:M SpMM."""
    R, K, Nc, V, M = 256, 512, 512, 64, 8
    Z = dev(synth.normal((R, K), 6, mean=-0.5), "bf16")
    B = dev(synth.normal((K, Nc), 7, std=0.02), "bf16")
    nv, mb, _ = nm.sizes(R, K, 2, M, V)
    vals = torch.empty((R, nv // R), dtype=torch.bfloat16, device="cuda")
    meta = torch.empty((R, mb // R), dtype=torch.uint8, device="cuda")
    cs = torch.empty((R // V, K // M, 4), dtype=torch.uint8, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")

    def step():
        nm.prune_act_venom(Z, V, M, apply_relu=True, values=vals, meta=meta, colsel=cs)
        nm.spmm_venom(vals, meta, cs, K, V, M, B, out=C)
    return step, [vals, meta, cs, C]


@pytest.mark.parametrize("make", [_up24, _train, _vnm], ids=["up24", "train", "vnm"])
def test_step_replays_from_a_hip_graph(make):
    step, outs = make()
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    # warm-up on a side stream (as torch asks before a capture), then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager step"
