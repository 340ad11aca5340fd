"""bench.py's host-side contract (CPU only): the multi-GPU refusal, the workload table, the
recorded-counter hash and a small oracle baseline."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_matmul_ffns_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_configs_cover_the_metric_workloads():
    names = [bench.HEADLINE] + bench.CONFIGS
    assert len(set(names)) == 6
    assert all(n in synth.WORKLOADS for n in names)
    kinds = {synth.WORKLOADS[n]["kind"] for n in names}
    assert {"spmm_nm", "spmm_venom", "train_step", "act_venom"} <= kinds


def test_source_hash_is_stable_and_path_free():
    h = bench._src_hash()
    assert h == bench._src_hash() and len(h) == 16
    from sparse_matmul_ffns_amd import build
    assert build.ROOT not in " ".join(build.FLAGS).replace(build.ROOT, "<repo>")


def test_kernel_source_sets():
    """Every file named for a kernel's counters exists, every quoted include of those files is in
    the set, and the per-kernel hashes differ from the whole-tree hash."""
    import re
    csrc = os.path.join(ROOT, "sparse_matmul_ffns_amd", "csrc")
    for kernel, files in bench.KERNEL_SOURCES.items():
        names = set(files) | set(bench.SHARED_SOURCES)
        for name in names:
            assert os.path.exists(os.path.join(csrc, name)), (kernel, name)
            for inc in re.findall(r'#include "([^"]+)"', open(os.path.join(csrc, name)).read()):
                assert inc in names or inc.endswith("include/nmsparse.h"), (kernel, name, inc)
        assert bench._src_hash(kernel) != bench._src_hash()


def test_cpu_baseline_small_case():
    r = bench.cpu_baseline("nm24_fp32_256x512x128")
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    json.dumps(r)
