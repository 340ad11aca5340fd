"""Throughput of the sparse FFN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the hot path over the workload's synthetic inputs
(already resident in HBM when the timed region starts):
  ffn_up_nm24_8192x2048x4096 (default): nm_prune_compress_transpose (the 2:4
      mask and the compressed weight in one pass over the weight, and the
      activations turned K-contiguous, in one launch) -> spmm_nm_t of a
      bf16 2:4 weight [8192 x 2048] ~ N(0, 0.02)
      with activations [2048 x 4096] ~ N(0, 1);
  ffn_down_vnm64_2_8_2048x8192x4096: prune_act_venom (V=64, M=8) -> spmm_venom;
  train_step_nm24_dmodel4096_dff16384_tok8192: nm_reprune_t_transpose_panels
      (the weight's 2:4 transpose re-pruned, in the panel layout, and X
      transposed, in one launch) -> spmm_nm_t (Y) -> sddmm_nm_dt (dW, and
      dY^T written from the SDDMM's LDS tiles) -> spmm_nm_t_panels (dX) (the
      weight's own prune and compress run once before timing);
  relu_act_vnm128_2_8_8192x16384x4096: prune_act_venom (ReLU, V=128, M=8) ->
      spmm_venom;
  nm24_fp32_256x512x128: the small fp32 case.
`value` is dense-equivalent TFLOP/s of the whole step (2 R K Nc per product,
pruned zeros counted as if dense).  `products` gives the same flops over the
event-timed durations of the step's matrix products alone (without the prune,
compress and transpose launches), beside `value`, never in its place.  The JSON
line also carries the roofline of the step's dominant kernel, timed with HIP
events on the stream it runs on, and the fp64 CPU oracle timed on the host
(rank 0, N = 1 only).

Without --workload the headline is the 2:4 up-projection, and `configs` adds
the same measurement (step time, dense-equivalent TFLOP/s, share of the bf16
peak, per-kernel times, roofline of the dominant kernel, oracle sample) for the
small fp32 case, the V:N:M down-projection, the double-pruned training step,
the ReLU V:N:M step and that step's backward (dZ at the kept activations and
dW_down).

A default run also measures the bf16 matrix rate the chip sustains under its
power limit (`sustained_mfma`: a chip-wide loop of independent matrix
instructions, no memory traffic) and reports every bf16 step against it
(`pct_of_sustained_bf16_dense`) beside the nominal peak.

Warm-up: the W untimed steps are repeated until at least one second of them
has run, so that the timed steps see settled GPU clocks.  `cold` reports, beside
`value`, the median of five single steps each run after 512 MiB have been
written over a scratch buffer (operands evicted from L2 and the last-level cache).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
WARMUP_MIN_S = 1.0            # minimum warm-up wall time (see main)
METRIC = "dense-equivalent TFLOP/s of 2:4 & V:N:M SpMM at FFN shapes; % of bf16 MFMA peak"
HEADLINE = "ffn_up_nm24_8192x2048x4096"
# the other workloads of the metric, measured beside the headline in a default run
CONFIGS = ["nm24_fp32_256x512x128", "ffn_down_vnm64_2_8_2048x8192x4096",
           "train_step_nm24_dmodel4096_dff16384_tok8192", "relu_act_vnm128_2_8_8192x16384x4096",
           "relu_act_vnm128_bwd_8192x16384x4096"]


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None, help=f"one workload (default: {HEADLINE} plus `configs`)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--single", action="store_true", help="measure the headline workload only (no `configs`)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of known size (to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return p.parse_args()


def copy_calibration(steps):
    """A plain 256 MiB device-to-device copy, `steps` times: the reference for the
    HBM byte counters (each launch reads and writes exactly 256 MiB)."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": steps}))


def sustained_mfma():
    """The bf16 matrix rate the chip sustains under its power limit, measured live: the library's
    probe (a chip-wide loop of independent matrix instructions on register operands that change
    every iteration, two waves per SIMD, no memory traffic), timed with HIP events on the stream it runs on, after a second of
    warm-up.  Dense v_mfma_f32_32x32x16_bf16 and 2:4 v_smfmac_f32_32x32x32_bf16 (dense-equivalent
    flops)."""
    import torch
    import sparse_matmul_ffns_amd as nm
    sink = torch.empty(512 * 256, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 4096
    res = {}
    for kind, key in ((0, "dense_bf16_tflops"), (1, "smfmac_2to4_dense_equivalent_tflops")):
        t0 = time.time()
        while time.time() - t0 < 1.0:
            nm.mfma_rate_probe(kind, iters, sink)
            torch.cuda.synchronize()
        best = 0.0
        for _ in range(5):
            e0.record()
            flops = nm.mfma_rate_probe(kind, iters, sink)
            e1.record()
            e1.synchronize()
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[key] = round(best, 1)
    res["how"] = ("chip-wide loop of independent bf16 matrix instructions on register operands that change every "
                  "iteration (random signs and significands; nm_mfma_rate_probe), 2 waves per SIMD, no memory traffic, "
                  "best of 5 launches after 1 s of warm-up")
    return res


def _dev(raw):
    import torch
    if raw.dtype == np.uint16:
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(raw).cuda()


# ---------------------------------------------------------------------------
# workloads: each returns (setup dict, list of (kernel name, callable), flops)
# ---------------------------------------------------------------------------

def _w_nm(w, dtype):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    R, K, Nc = w["R"], w["K"], w["Nc"]
    A = _dev(synth.normal((R, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"], dtype))
    B = _dev(synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"], dtype))
    mask = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    nv, mb, _ = nm.sizes(R, K, 2, 4)
    vals = torch.empty((R, nv // R), dtype=A.dtype, device="cuda")
    meta = torch.empty((R, mb // R), dtype=torch.uint8, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")
    if dtype == "bf16":
        # one launch selects and compresses the weight (the mask and the values + metadata,
        # byte-identical to nm_prune then nm_compress) and turns the activations K-contiguous
        # (nm_transpose); spmm_nm_t then streams both operands into LDS as whole rows
        Bt = torch.empty((Nc, K), dtype=B.dtype, device="cuda")
        steps = [
            ("nm_prune_compress_transpose",
             lambda: nm.nm_prune_compress_transpose(A, B, 2, 4, mask=mask, values=vals, meta=meta, Bt=Bt)),
            ("spmm_nm_t", lambda: nm.spmm_nm_t(vals, meta, K, Bt, out=C)),
        ]
        kernel = "spmm_nm_t"
    else:
        steps = [("nm_prune_compress", lambda: nm.nm_prune_compress(A, 2, 4, mask=mask, values=vals, meta=meta)),
                 ("spmm_nm", lambda: nm.spmm_nm(vals, meta, K, B, out=C))]
        kernel = "spmm_nm"
    flops = {kernel: 2.0 * R * K * Nc}
    algo = {kernel: ("mfma", R * (K // 2) * Nc * 2.0)}
    return steps, flops, algo, kernel


def _w_lowrank(w):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    R, K, Nc, r = w["R"], w["K"], w["Nc"], w["rank"]
    A = _dev(synth.normal((R, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"]))
    B = _dev(synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"]))
    U = _dev(synth.normal((R, r), w["U"]["seed"], w["U"]["mean"], w["U"]["std"]))
    Vt = _dev(synth.normal((r, K), w["Vt"]["seed"], w["Vt"]["mean"], w["Vt"]["std"]))
    mask = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    nv, mb, _ = nm.sizes(R, K, 2, 4)
    vals = torch.empty((R, nv // R), dtype=A.dtype, device="cuda")
    meta = torch.empty((R, mb // R), dtype=torch.uint8, device="cuda")
    Bt = torch.empty((Nc, K), dtype=B.dtype, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")
    Tt = torch.empty((Nc, r), dtype=torch.float32, device="cuda")
    # the 2:4 step with a low-rank adapter: the adapter's inner activations (one launch), then the
    # SpMM with the adapter term added to its accumulators
    steps = [
        ("nm_prune_compress_transpose",
         lambda: nm.nm_prune_compress_transpose(A, B, 2, 4, mask=mask, values=vals, meta=meta, Bt=Bt)),
        ("spmm_nm_t_lowrank", lambda: nm.spmm_nm_t_lowrank(vals, meta, K, Bt, U, Vt, out=C, Tt=Tt)),
    ]
    # dense-equivalent flops of the adapted layer: those of the dense [R x K] weight it stands for
    flops = {"spmm_nm_t_lowrank": 2.0 * R * K * Nc}
    algo = {"spmm_nm_t_lowrank": ("mfma", R * (K // 2) * Nc * 2.0 + 2.0 * r * K * Nc + 2.0 * R * r * Nc)}
    return steps, flops, algo, "spmm_nm_t_lowrank"


def _w_general(w):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    R, K, Nc, N, M = w["R"], w["K"], w["Nc"], w["N"], w["M"]
    A = _dev(synth.normal((R, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"]))
    B = _dev(synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"]))
    mask = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    nv, mb, _ = nm.sizes(R, K, N, M)
    vals = torch.empty((R, nv // R), dtype=A.dtype, device="cuda")
    meta = torch.empty((R, mb // R), dtype=torch.uint8, device="cuda")
    Bt = torch.empty((Nc, K), dtype=B.dtype, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")
    work = torch.empty(nm.general_work_bytes(A.dtype, R, K, N, M), dtype=torch.uint8, device="cuda")
    # prune + compress to N:M and the activations' transpose, then the product (for N <= 2 the
    # matrix is rewritten in 2:4 form in `work` and multiplied by the 2:4 SpMM)
    steps = [
        ("nm_prune_compress_transpose",
         lambda: nm.nm_prune_compress_transpose(A, B, N, M, mask=mask, values=vals, meta=meta, Bt=Bt)),
        ("spmm_nm_general", lambda: nm.spmm_nm_general(vals, meta, K, N, M, Bt, out=C, work=work)),
    ]
    flops = {"spmm_nm_general": 2.0 * R * K * Nc}
    algo = {"spmm_nm_general": ("mfma", 2.0 * R * (K // M * N) * Nc)}
    return steps, flops, algo, "spmm_nm_general"


def _w_block(w):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    dm, dff, T, V, M = w["d_model"], w["d_ff"], w["tokens"], w["V"], w["M"]
    W = _dev(synth.normal((dff, dm), w["W"]["seed"], w["W"]["mean"], w["W"]["std"]))
    Xt = _dev(synth.normal((T, dm), w["X"]["seed"], w["X"]["mean"], w["X"]["std"]))
    Wd = _dev(synth.normal((dff, dm), w["W_down"]["seed"], w["W_down"]["mean"], w["W_down"]["std"]))
    mask = torch.empty((dff, dm), dtype=torch.uint8, device="cuda")
    vals = torch.empty((dff, dm // 2), dtype=W.dtype, device="cuda")
    meta = torch.empty((dff, dm // 8), dtype=torch.uint8, device="cuda")
    hT = torch.empty((dff, T), dtype=W.dtype, device="cuda")
    h = torch.empty((T, dff), dtype=W.dtype, device="cuda")
    nv, mb, cb = nm.sizes(T, dff, 2, M, V)
    hv = torch.empty((T, nv // T), dtype=W.dtype, device="cuda")
    hm = torch.empty((T, mb // T), dtype=torch.uint8, device="cuda")
    hc = torch.empty((T // V, dff // M, 4), dtype=torch.uint8, device="cuda")
    Y = torch.empty((T, dm), dtype=torch.float32, device="cuda")
    # the FFN block forward from its parts: the weight's 2:4 prune + compress, the up-projection
    # (bf16 output, [d_ff x tokens]), the activations made token-major, ReLU + V:N:M prune, and the
    # V:N:M down-projection
    if w["kind"] == "ffn_block_fused":
        # the up-projection prunes its activations in its epilogue: h is never stored
        del hT, h
        steps = [
            ("nm_prune_compress", lambda: nm.nm_prune_compress(W, 2, 4, mask=mask, values=vals, meta=meta)),
            ("spmm_nm_t_relu_venom", lambda: nm.spmm_nm_t_relu_venom(vals, meta, dm, Xt, V, M, h_values=hv,
                                                                     h_meta=hm, h_colsel=hc)),
            ("spmm_venom_down", lambda: nm.spmm_venom(hv, hm, hc, dff, V, M, Wd, out=Y)),
        ]
        g = 2.0 * dff * dm * T
        flops = {"spmm_nm_t_relu_venom": g, "spmm_venom_down": g}
        algo = {"spmm_nm_t_relu_venom": ("mfma", g / 2), "spmm_venom_down": ("mfma", g / 4)}
        return steps, flops, algo, "spmm_venom_down"
    steps = [
        ("nm_prune_compress", lambda: nm.nm_prune_compress(W, 2, 4, mask=mask, values=vals, meta=meta)),
        ("spmm_nm_t_up", lambda: nm.spmm_nm_t(vals, meta, dm, Xt, out=hT)),
        ("nm_transpose_h", lambda: nm.transpose(hT, out=h)),
        ("prune_act_venom", lambda: nm.prune_act_venom(h, V, M, apply_relu=True, values=hv, meta=hm, colsel=hc)),
        ("spmm_venom_down", lambda: nm.spmm_venom(hv, hm, hc, dff, V, M, Wd, out=Y)),
    ]
    g = 2.0 * dff * dm * T
    flops = {"spmm_nm_t_up": g, "spmm_venom_down": g}
    algo = {"spmm_nm_t_up": ("mfma", g / 2), "spmm_venom_down": ("mfma", g / 4)}
    return steps, flops, algo, "spmm_venom_down"


def _w_venom(w, relu):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    R, K, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
    a = w["Z"] if relu else w["A"]
    b = w["W"] if relu else w["B"]
    Z = _dev(synth.normal((R, K), a["seed"], a["mean"], a["std"]))
    B = _dev(synth.normal((K, Nc), b["seed"], b["mean"], b["std"]))
    nv, mb, cb = nm.sizes(R, K, 2, M, V)
    vals = torch.empty((R, nv // R), dtype=Z.dtype, device="cuda")
    meta = torch.empty((R, mb // R), dtype=torch.uint8, device="cuda")
    colsel = torch.empty((R // V, K // M, 4), dtype=torch.uint8, device="cuda")
    C = torch.empty((R, Nc), dtype=torch.float32, device="cuda")
    steps = [
        ("prune_act_venom", lambda: nm.prune_act_venom(Z, V, M, apply_relu=relu, values=vals, meta=meta,
                                                       colsel=colsel)),
        ("spmm_venom", lambda: nm.spmm_venom(vals, meta, colsel, K, V, M, B, out=C)),
    ]
    flops = {"spmm_venom": 2.0 * R * K * Nc}
    algo = {"spmm_venom": ("mfma", R * (K // M * 2) * Nc * 2.0),
            "prune_act_venom": ("hbm", R * K * 2 + nv * 2 + mb + cb)}
    return steps, flops, algo, "spmm_venom"


def _w_venom_bwd(w):
    """Backward of the ReLU V:N:M down-projection: dZ at the kept activations (and dY^T), then
    dW_down = h_s^T dY.  h_s comes from the forward's prune (not timed)."""
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    T, F, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
    Z = _dev(synth.normal((T, F), w["Z"]["seed"], w["Z"]["mean"], w["Z"]["std"]))
    Wd = _dev(synth.normal((F, Nc), w["W"]["seed"], w["W"]["mean"], w["W"]["std"]))
    dY = _dev(synth.normal((T, Nc), w["dY"]["seed"], w["dY"]["mean"], w["dY"]["std"]))
    hv, hm, hc = nm.prune_act_venom(Z, V, M, apply_relu=True)
    del Z
    dz = torch.empty((T, F // M * 2), dtype=torch.float32, device="cuda")
    dYt = torch.empty((Nc, T), dtype=dY.dtype, device="cuda")
    dW = torch.empty((F, Nc), dtype=torch.float32, device="cuda")
    work = torch.empty(nm.venom_tn_work_bytes(dY.dtype, T, F), dtype=torch.uint8, device="cuda")
    steps = [
        ("sddmm_venom", lambda: nm.sddmm_venom(dY, Wd, hv, hm, hc, V, M, apply_relu=True, out=dz, dYt=dYt)),
        ("spmm_venom_tn", lambda: nm.spmm_venom_tn(hv, hm, hc, F, V, M, dYt, out=dW, work=work)),
    ]
    g = 2.0 * T * F * Nc
    flops = {"sddmm_venom": g, "spmm_venom_tn": g}
    algo = {"sddmm_venom": ("mfma", g / M * 4), "spmm_venom_tn": ("mfma", g)}
    return steps, flops, algo, "spmm_venom_tn"


def _w_train(w):
    import torch
    import sparse_matmul_ffns_amd as nm
    from sparse_matmul_ffns_amd import synth
    dm, dff, T = w["d_model"], w["d_ff"], w["tokens"]
    W = _dev(synth.normal((dff, dm), w["W"]["seed"], w["W"]["mean"], w["W"]["std"]))
    X = _dev(synth.normal((dm, T), w["X"]["seed"], w["X"]["mean"], w["X"]["std"]))
    dY = _dev(synth.normal((dff, T), w["dY"]["seed"], w["dY"]["mean"], w["dY"]["std"]))
    mask = nm.nm_prune(W)
    vals, meta = nm.nm_compress(W, mask)
    del mask
    vt = torch.empty((dm, dff // 2), dtype=W.dtype, device="cuda")
    mt = torch.empty((dm, dff // 8), dtype=torch.uint8, device="cuda")
    Y = torch.empty((dff, T), dtype=torch.float32, device="cuda")
    dX = torch.empty((dm, T), dtype=torch.float32, device="cuda")
    dW = torch.empty((dff, dm // 2), dtype=torch.float32, device="cuda")
    Xt = torch.empty((T, dm), dtype=X.dtype, device="cuda")
    dYt = torch.empty((T, dff), dtype=dY.dtype, device="cuda")
    # dW comes before dX: the SDDMM stages every tile of dY through LDS and writes dY^T from there
    # (sddmm_nm_dt), which the dX product then reads K-contiguous.  The re-pruned transpose is
    # written in the panel layout, which the dX product (K = d_ff: 256 steps per tile) reads with
    # four waves two steps ahead
    steps = [
        ("nm_reprune_t_transpose_panels",
         lambda: nm.nm_reprune_t_transpose_panels(vals, meta, dff, dm, X, values_t=vt, meta_t=mt, Xt=Xt)),
        ("spmm_nm_t_fwd", lambda: nm.spmm_nm_t(vals, meta, dm, Xt, out=Y)),
        ("sddmm_nm_dt", lambda: nm.sddmm_nm(dY, X, meta, out=dW, Dt=dYt)),
        ("spmm_nm_t_panels_dx", lambda: nm.spmm_nm_t_panels(vt, mt, dm, dff, dYt, out=dX)),
    ]
    g = 2.0 * dff * dm * T
    flops = {"spmm_nm_t_fwd": g, "spmm_nm_t_panels_dx": g, "sddmm_nm_dt": g}
    algo = {"spmm_nm_t_fwd": ("mfma", g / 2), "spmm_nm_t_panels_dx": ("mfma", g / 2), "sddmm_nm_dt": ("mfma", g),
            "nm_reprune_t_transpose_panels": ("hbm", 2 * (dff * dm // 2 * 2 + dff * dm // 8) + 2 * dm * T * 2)}
    return steps, flops, algo, "sddmm_nm_dt"


def build_workload(name):
    from sparse_matmul_ffns_amd import synth
    w = synth.WORKLOADS[name]
    if w["kind"] == "spmm_nm":
        return _w_nm(w, w["dtype"])
    if w["kind"] == "spmm_nm_lowrank":
        return _w_lowrank(w)
    if w["kind"] == "spmm_nm_general":
        return _w_general(w)
    if w["kind"] in ("ffn_block", "ffn_block_fused"):
        return _w_block(w)
    if w["kind"] == "spmm_venom":
        return _w_venom(w, relu=False)
    if w["kind"] == "act_venom":
        return _w_venom(w, relu=True)
    if w["kind"] == "act_venom_bwd":
        return _w_venom_bwd(w)
    return _w_train(w)


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, host cores)
# ---------------------------------------------------------------------------

def cpu_baseline(name):
    from oracle import nm_oracle as O
    from sparse_matmul_ffns_amd import synth
    w = synth.WORKLOADS[name]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if w["kind"] in ("spmm_nm",):
        R, K, Nc = w["R"], w["K"], w["Nc"]
        rows = R
        A = synth.normal((rows, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"], w["dtype"])
        B = synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"], w["dtype"])
        t0 = time.perf_counter()
        mask = O.prune_nm(A, w["dtype"], 2, 4)
        v, m, _ = O.compress_nm(A, mask, 2, 4)
        O.spmm_nm(v, m, rows, K, B, w["dtype"])
        dt = time.perf_counter() - t0
        fl = 2.0 * rows * K * Nc
        sample = f"whole workload, one step: prune + compress of the [{R}x{K}] weight, fp64 decompress-and-dgemm with the [{K}x{Nc}] operand"
    elif w["kind"] == "spmm_nm_general":
        R, K, Nc, N, M = w["R"], w["K"], w["Nc"], w["N"], w["M"]
        A = synth.normal((R, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"])
        B = synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"])
        t0 = time.perf_counter()
        v, m, _ = O.compress_nm(A, O.prune_nm(A, "bf16", N, M), N, M)
        O.spmm_nm_general(v, m, R, K, N, M, B, "bf16")
        dt = time.perf_counter() - t0
        fl = 2.0 * R * K * Nc
        sample = (f"whole workload, one step: {N}:{M} prune + compress of the [{R}x{K}] weight, fp64 "
                  f"decompress-and-dgemm with the [{K}x{Nc}] operand")
    elif w["kind"] in ("ffn_block", "ffn_block_fused"):
        dm, dff, T, V, M = w["d_model"], w["d_ff"], w["tokens"], w["V"], w["M"]
        W = synth.normal((dff, dm), w["W"]["seed"], w["W"]["mean"], w["W"]["std"])
        Xt = synth.normal((V, dm), w["X"]["seed"], w["X"]["mean"], w["X"]["std"])   # the first V tokens
        Wd = synth.normal((dff, dm), w["W_down"]["seed"], w["W_down"]["mean"], w["W_down"]["std"])
        t0 = time.perf_counter()
        v, m, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
        hT = O.spmm_nm(v, m, dff, dm, np.ascontiguousarray(Xt.T), "bf16")         # [d_ff x V] in fp64
        hv, hm, hc, _, _ = O.prune_venom(O.encode_bf16(hT.T), "bf16", V, M, True)
        O.spmm_venom(hv, hm, hc, V, dff, V, M, Wd, "bf16")
        dt = time.perf_counter() - t0
        fl = 2 * 2.0 * dff * dm * V
        sample = (f"{V} of {T} tokens (one V-block): the weight's 2:4 prune + compress, the fp64 up-projection, "
                  f"bf16 rounding, ReLU + V:N:M prune and the fp64 down-projection")
    elif w["kind"] == "spmm_nm_lowrank":
        R, K, Nc, r = w["R"], w["K"], w["Nc"], w["rank"]
        A = synth.normal((R, K), w["A"]["seed"], w["A"]["mean"], w["A"]["std"])
        B = synth.normal((K, Nc), w["B"]["seed"], w["B"]["mean"], w["B"]["std"])
        U = synth.normal((R, r), w["U"]["seed"], w["U"]["mean"], w["U"]["std"])
        Vt = synth.normal((r, K), w["Vt"]["seed"], w["Vt"]["mean"], w["Vt"]["std"])
        t0 = time.perf_counter()
        v, m, _ = O.compress_nm(A, O.prune_nm(A, "bf16", 2, 4), 2, 4)
        O.spmm_nm_lowrank(v, m, R, K, B, U, Vt, "bf16")
        dt = time.perf_counter() - t0
        fl = 2.0 * R * K * Nc
        sample = (f"whole workload, one step: prune + compress of the [{R}x{K}] weight, fp64 decompress-and-dgemm "
                  f"with the [{K}x{Nc}] operand plus the rank-{r} adapter")
    elif w["kind"] == "act_venom_bwd":
        # one V-block of tokens through both backward products (the oracle's own V:N:M prune of
        # that block of activations first)
        T, F, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
        Z = synth.normal((V, F), w["Z"]["seed"], w["Z"]["mean"], w["Z"]["std"])
        Wd = synth.normal((F, Nc), w["W"]["seed"], w["W"]["mean"], w["W"]["std"])
        dY = synth.normal((V, Nc), w["dY"]["seed"], w["dY"]["mean"], w["dY"]["std"])
        hv, hm, hc, _, _ = O.prune_venom(Z, "bf16", V, M, True)
        t0 = time.perf_counter()
        O.sddmm_venom(dY, Wd, hv, hm, hc, V, F, V, M, "bf16", True)
        O.spmm_venom_tn(hv, hm, hc, V, F, V, M, dY, "bf16")
        dt = time.perf_counter() - t0
        fl = 2 * 2.0 * V * F * Nc
        sample = (f"{V} of {T} tokens (one V-block, pruned by the oracle first, not timed): dZ at the kept "
                  f"activations and dW_down's share of that block, fp64")
    elif w["kind"] == "train_step":
        # a slice of the d_ff rows of the layer (whole 2:4 groups of W_s^T): W's prune + compress,
        # Y for those rows, the re-pruned transpose of the slice and its share of dX, dW at the
        # slice's survivors -- all three products of the step on 1/64 of the d_ff dimension
        dm, dff, T = w["d_model"], w["d_ff"], w["tokens"]
        rows = 1024
        W = synth.normal((rows, dm), w["W"]["seed"], w["W"]["mean"], w["W"]["std"])
        X = synth.normal((dm, T), w["X"]["seed"], w["X"]["mean"], w["X"]["std"])
        dY = synth.normal((rows, T), w["dY"]["seed"], w["dY"]["mean"], w["dY"]["std"])
        t0 = time.perf_counter()
        v, m, _ = O.compress_nm(W, O.prune_nm(W, "bf16", 2, 4), 2, 4)
        O.spmm_nm(v, m, rows, dm, X, "bf16")                                   # Y rows
        vt, mt = O.reprune_t(v, m, rows, dm, "bf16")                             # W_ds^T [dm x rows]
        O.spmm_nm(vt, mt, dm, rows, dY, "bf16")                                  # the slice's share of dX
        O.sddmm_nm(dY, X, m, rows, dm, "bf16")                                   # dW at the survivors
        dt = time.perf_counter() - t0
        fl = 3 * 2.0 * rows * dm * T
        sample = (f"{rows} of {dff} d_ff rows (the first rows of W and dY, the whole X): "
                  f"2:4 prune + compress, fp64 Y, re-prune of the transposed slice and its share of dX, dW at the "
                  f"survivors (1/{dff // rows} of each product)")
    else:
        R, K, Nc, V, M = w["R"], w["K"], w["Nc"], w["V"], w["M"]
        rows = min(R, 2048)
        a = w.get("Z") or w.get("A")
        b = w.get("W") or w.get("B")
        A = synth.normal((rows, K), a["seed"], a["mean"], a["std"])
        B = synth.normal((K, Nc), b["seed"], b["mean"], b["std"])
        t0 = time.perf_counter()
        v, m, c, _, _ = O.prune_venom(A, "bf16", V, M, w["kind"] == "act_venom")
        O.spmm_venom(v, m, c, rows, K, V, M, B, "bf16")
        dt = time.perf_counter() - t0
        fl = 2.0 * rows * K * Nc
        sample = f"{rows} of {R} rows: V:N:M prune + fp64 decompress-and-dgemm with the full [{K}x{Nc}] operand"
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


# ---------------------------------------------------------------------------
# counters recorded with rocprofv3 (profiles/), valid while the kernel source is unchanged
# ---------------------------------------------------------------------------

# the kernel sources behind each step name whose counters are recorded: the file of the kernel and
# of the launch routine that picks it (besides the files every kernel shares)
KERNEL_SOURCES = {
    "spmm_nm_t": ["spmm_nt.hip", "spmm.hip"],
    "spmm_nm_t_fwd": ["spmm_nt.hip", "spmm.hip"],
    "spmm_nm_t_dx": ["spmm_nt.hip", "spmm.hip"],
    "spmm_nm_t_up": ["spmm_nt.hip", "spmm.hip"],
    "spmm_nm_t_lowrank": ["spmm_nt.hip", "lowrank.hip"],
    "spmm_nm_t_relu_venom": ["spmm_nt.hip"],
    "spmm_nm_general": ["general.hip", "spmm_nt.hip", "spmm.hip", "sddmm.hip"],
    "spmm_nm": ["spmm.hip", "spmm_dma.hip"],
    "spmm_venom": ["spmm.hip", "spmm_vnm.hip", "spmm_dma.hip"],
    "spmm_venom_down": ["spmm.hip", "spmm_vnm.hip", "spmm_dma.hip"],
    "sddmm_nm_dt": ["sddmm.hip"],
    "sddmm_venom": ["sddmm.hip", "venom_bwd.hip"],
    "spmm_venom_tn": ["sddmm.hip", "venom_bwd.hip"],
    "prune_act_venom": ["venom.hip"],
    "nm_reprune_t": ["reprune.hip"],
    "nm_reprune_t_transpose": ["reprune.hip"],
    "nm_reprune_t_transpose_panels": ["reprune.hip"],
    "spmm_nm_t_panels_dx": ["spmm_w4.hip"],
}
SHARED_SOURCES = ["api.cpp", "common.hpp", "dma.hpp", "launch.hpp", "prep_bodies.hpp"]


def _src_hash(kernel=None):
    """Hash of the sources a kernel is built from (its own file and its launch routine, the shared
    headers, the C ABI, the public header) and of the build flags: recorded counters describe the
    code built from exactly these.  Without a kernel (or for one not listed), every source file."""
    from sparse_matmul_ffns_amd import build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_matmul_ffns_amd", "csrc")
    names = sorted(os.listdir(csrc))
    if kernel in KERNEL_SOURCES:
        names = sorted(set(KERNEL_SOURCES[kernel]) | set(SHARED_SOURCES))
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "nmsparse.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(build.FLAGS).replace(build.ROOT, "<repo>").encode())
    return h.hexdigest()[:16]


def recorded_counter(workload, kernel, key):
    """A per-launch figure (`hbm_bytes_per_launch`, `mfma_busy_pct`) from the committed rocprofv3
    --pmc summary of the kernel on the workload, or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != _src_hash(kernel):
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


COLD_RUNS = 5
COLD_FLUSH_BYTES = 512 << 20


def measure(workload, steps_n, warmup_n, with_cpu):
    """One workload: warm-up, K timed steps, K event-timed steps (per-kernel durations), cold steps,
    and the oracle sample; returns the figures as a dict."""
    import torch
    steps, flops, algo, dominant = build_workload(workload)
    torch.cuda.synchronize()

    # W untimed warm-up steps, continued until at least WARMUP_MIN_S of them have run: from idle the
    # GPU needs a few hundred milliseconds of load before its clocks settle, and steps timed
    # earlier run up to 20% slower
    t_w = time.perf_counter()
    done = 0
    while done < warmup_n or time.perf_counter() - t_w < WARMUP_MIN_S:
        for _, fn in steps:
            fn()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # timed region: exactly K steps, launched back to back with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps_n):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel durations for the roofline: a second pass of K steps with HIP events recorded on
    # the launch stream between the kernels (the events themselves leave small gaps, which is why
    # they stay out of the timed region)
    stream = torch.cuda.current_stream()
    names = [n for n, _ in steps]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(steps_n)]
    for st in range(steps_n):
        ev[st][0].record(stream)
        for i, (_, fn) in enumerate(steps):
            fn()
            ev[st][i + 1].record(stream)
    torch.cuda.synchronize()
    per_kernel_ms = {n: float(np.mean([ev[st][i].elapsed_time(ev[st][i + 1]) for st in range(steps_n)]))
                     for i, n in enumerate(names)}

    # cold steps (reported beside, not as `value`): before each, 512 MiB written over a scratch
    # buffer push the step's operands out of L2 and the 256 MB last-level cache; the step is then
    # timed alone between two events
    flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    cold_ms = []
    for i in range(COLD_RUNS):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _, fn in steps:
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(e0.elapsed_time(e1))
    del flush, steps
    torch.cuda.empty_cache()
    ms_per_step = elapsed * 1e3 / steps_n
    total_flops = sum(flops.values())
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    # the step's matrix products alone (their event-timed durations, without the prune, compress
    # and transpose launches around them): beside `value`, never in its place
    prod_ms = sum(per_kernel_ms[n] for n in flops)
    prod_tflops = total_flops / (prod_ms * 1e-3) / 1e12

    from sparse_matmul_ffns_amd import synth
    w = synth.WORKLOADS[workload]
    bound, per_launch = algo[dominant]
    t_dom = per_kernel_ms[dominant] * 1e-3
    if bound == "mfma":
        achieved, unit = per_launch / t_dom / 1e12, "TFLOP/s"
        peak = PEAK_FP32_MFMA_TFLOPS if w["dtype"] == "f32" else PEAK_BF16_TFLOPS
    else:
        achieved, peak, unit = per_launch / t_dom / 1e9, PEAK_HBM_GBS, "GB/s"
    res = {
        "workload": workload,
        "ms_per_step": round(ms_per_step, 5),
        "value": round(value, 2),
        "steps": steps_n,
        "warmup_steps_run": done,
        "dtype": "bf16" if w["dtype"] == "bf16" else "f32",
        "kernels": names,
        "pct_of_bf16_peak_dense_equivalent": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "per_kernel_us": {n: round(v * 1e3, 2) for n, v in per_kernel_ms.items()},
        "products": {"kernels": list(flops), "us": round(prod_ms * 1e3, 2),
                     "dense_equiv_tflops": round(prod_tflops, 2),
                     "pct_of_bf16_peak": round(100 * prod_tflops / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": recorded_counter(workload, dominant, "hbm_bytes_per_launch"),
                     "mfma_busy_pct": recorded_counter(workload, dominant, "mfma_busy_pct"),
                     "counters": "recorded: rocprofv3 --pmc of the same sources and build flags "
                                 f"(profiles/{dominant}_{workload}_pmc.txt); null when they differ"},
        "cold": {"ms_per_step": round(float(np.median(cold_ms)), 5),
                 "value": round(total_flops / (float(np.median(cold_ms)) * 1e-3) / 1e12, 2),
                 "runs": COLD_RUNS, "flush_bytes": COLD_FLUSH_BYTES},
    }
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(workload)
    return res


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU "
              "component", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    workload = args.workload or HEADLINE
    head = measure(workload, args.steps, args.warmup, not args.no_cpu)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded normal inputs of the workload's shapes; no dataset or trained weights)",
        "config": {"workload": workload, "kernels": head["kernels"],
                   "pct_of_bf16_peak_dense_equivalent": head["pct_of_bf16_peak_dense_equivalent"]},
        "per_kernel_us": head["per_kernel_us"],
        "products": head["products"],
        "roofline": head["roofline"],
        "cold": head["cold"],
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if args.workload is None and not args.single:
        out["configs"] = {}
        for name in CONFIGS:
            r = measure(name, args.steps, args.warmup, not args.no_cpu)
            r.pop("workload")
            out["configs"][name] = r
        # the same figures against the matrix rate the chip sustains (measured last, so that its
        # full-power loop does not warm the chip for the workloads)
        sus = sustained_mfma()
        out["sustained_mfma"] = sus
        dense = sus["dense_bf16_tflops"]
        out["config"]["pct_of_sustained_bf16_dense"] = round(100.0 * out["value"] / dense, 2)
        for r in out["configs"].values():
            if r.get("dtype") == "bf16":
                r["pct_of_sustained_bf16_dense"] = round(100.0 * r["value"] / dense, 2)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
