"""The library's calls from several host threads at once.

The library keeps no state between calls (the text of the last HIP error is thread-local), so
calls from different host threads, each on its own stream, may interleave freely.  Two threads
run different steps twenty times each on their own streams while the other runs; each thread's
outputs must equal those of the same step run alone.
"""

import threading

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
    R, K, Nc = 512, 1024, 768
    W, X = dev(synth.normal((R, K), 61, std=0.02), "bf16"), dev(synth.normal((K, Nc), 62), "bf16")
    outs = [torch.empty((R, K), dtype=torch.uint8, device="cuda"),
            torch.empty((R, K // 2), dtype=torch.bfloat16, device="cuda"),
            torch.empty((R, K // 8), dtype=torch.uint8, device="cuda"),
            torch.empty((Nc, K), dtype=torch.bfloat16, device="cuda"),
            torch.empty((R, Nc), dtype=torch.float32, device="cuda")]
    mask, vals, meta, Bt, C = outs

    def step():
        nm.nm_prune_compress_transpose(W, X, mask=mask, values=vals, meta=meta, Bt=Bt)
        nm.spmm_nm_t(vals, meta, K, Bt, out=C)
    return step, outs


def _vnm():
    R, K, Nc, V, M = 256, 1024, 512, 64, 8
    Z = dev(synth.normal((R, K), 63, mean=-0.5), "bf16")
    B = dev(synth.normal((K, Nc), 64, std=0.02), "bf16")
    nv, mb, _ = nm.sizes(R, K, 2, M, V)
    outs = [torch.empty((R, nv // R), dtype=torch.bfloat16, device="cuda"),
            torch.empty((R, mb // R), dtype=torch.uint8, device="cuda"),
            torch.empty((R // V, K // M, 4), dtype=torch.uint8, device="cuda"),
            torch.empty((R, Nc), dtype=torch.float32, device="cuda")]
    vals, meta, cs, C = outs

    def step():
        nm.prune_act_venom(Z, V, M, apply_relu=True, values=vals, meta=meta, colsel=cs)
        nm.spmm_venom(vals, meta, cs, K, V, M, B, out=C)
    return step, outs


def test_calls_from_two_host_threads():
    jobs = [_up24(), _vnm()]
    refs = []
    for step, outs in jobs:
        step()
        torch.cuda.synchronize()
        refs.append([o.clone() for o in outs])
        for o in outs:
            o.zero_()
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(i):
        try:
            step, outs = jobs[i]
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(20):
                    step()
            s.synchronize()
            for j, (o, r) in enumerate(zip(outs, refs[i])):
                if not torch.equal(o, r):
                    errors.append(f"thread {i}: output {j} differs from the step run alone")
        except Exception as e:   # reported below, with the thread it came from
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
