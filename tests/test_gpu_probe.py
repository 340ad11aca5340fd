"""The matrix-rate probe (a measurement aid of the benchmark) runs, reports the flops of its launch,
and writes a finite value for every thread."""

import pytest
import torch

import sparse_matmul_ffns_amd as nm
from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,per_instr", [(0, 2 * 32 * 32 * 16), (1, 2 * 32 * 32 * 32)])
def test_mfma_rate_probe(kind, per_instr):
    require_gpu()
    sink = torch.full((512 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = nm.mfma_rate_probe(kind, 16, sink)
    torch.cuda.synchronize()
    assert flops == per_instr * 8 * 16 * 512 * 4
    assert bool(torch.isfinite(sink).all())
