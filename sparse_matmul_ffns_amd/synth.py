"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no pruning, compression or matmul arithmetic: it only draws
normal samples with numpy's PCG64 generator, rounds them to fp32 and then to
bf16 (round to nearest even on the fp32 bit pattern), and hands out raw bit
arrays.  Both sides of every parity check read the same bytes.

Workloads (feed-forward-network shapes, N(mu, sigma) entries):
  * 2:4 fp32 weight [256 x 512] with a [512 x 128] dense operand,
  * 2:4 bf16 up-projection weight [8192 x 2048], activations [2048 x 4096],
  * V:N:M (V=64, M=8) bf16 down-projection weight [2048 x 8192], activations
    [8192 x 4096],
  * one 2:4 training step with d_model 4096, d_ff 16384, 8192 tokens,
  * ReLU activations [8192 x 16384] ~ N(-0.5, 1) pruned V:N:M (V=128, M=8)
    times a dense down-projection weight [16384 x 4096].
Seeds: workload c draws tensor t from PCG64(1000*c + t), t = 0 for the sparse
operand, 1 for the dense operand, 2 for the backward gradient.
"""

from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns.

    Finite inputs only: adding 0x7FFF plus the lowest kept bit cannot carry
    out of 32 bits for any finite fp32 pattern.
    """
    u = np.array(x, dtype=np.float32, copy=True).reshape(-1).view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16).reshape(np.shape(x))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(shape, seed: int, mean: float = 0.0, std: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """N(mean, std) samples: raw uint16 bf16 bits (dtype 'bf16') or float32 ('f32').

    float64 standard normals from PCG64(seed), scaled, rounded to fp32 and (for
    bf16) to bf16; drawn in chunks, which yields the same stream as one draw.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    chunk = 1 << 22
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(size=e - s, dtype=np.float64)
        x *= std
        x += mean
        y = x.astype(np.float32)
        out[s:e] = f32_to_bf16_bits(y) if dtype == "bf16" else y
    return out.reshape(shape)


def small_ints(shape, seed: int, lo: int = -8, hi: int = 8, dtype: str = "bf16") -> np.ndarray:
    """Uniform integers in [lo, hi] (exact in bf16 and fp32): raw bits or float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# Counter-based integers for operands too large to draw on the host: entry (i, j) depends on i, j and
# the seed only, so a device fills the whole matrix and the host regenerates any rows or columns it
# samples.  h = (i * 0x9E3779B1 + j * 0x85EBCA77 + seed * 0xC2B2AE3D) mod 2^32, then the
# lowbias32 finalizer (h ^= h >> 16; h *= 0x7FEB352D; h ^= h >> 15; h *= 0x846CA68B; h ^= h >> 16,
# all mod 2^32), and the entry is h mod (2 span + 1) - span.
_HASH_I, _HASH_J, _HASH_S = 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D
_MASK32 = 0xFFFFFFFF


def hashed_ints(rows, cols, seed: int, span: int = 3) -> np.ndarray:
    """Entries (i, j) for i in `rows`, j in `cols` (1-D index arrays): integers in [-span, span] as
    bf16 bit patterns, shape [len(rows), len(cols)]."""
    i = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    j = np.asarray(cols, dtype=np.uint64).reshape(1, -1)
    m = np.uint64(_MASK32)
    h = (i * np.uint64(_HASH_I) + j * np.uint64(_HASH_J) + np.uint64((seed * _HASH_S) & _MASK32)) & m
    h ^= h >> np.uint64(16)
    h = (h * np.uint64(0x7FEB352D)) & m
    h ^= h >> np.uint64(15)
    h = (h * np.uint64(0x846CA68B)) & m
    h ^= h >> np.uint64(16)
    v = (h % np.uint64(2 * span + 1)).astype(np.int64) - span
    return f32_to_bf16_bits(v.astype(np.float32))


def hashed_ints_torch(rows, cols, seed: int, span: int = 3, block: int = 1 << 24):
    """hashed_ints on the device of `rows` (1-D int64 torch tensors): a torch.bfloat16 matrix
    [len(rows), len(cols)], built in pieces of about `block` entries.  The arithmetic is int64 with
    the low 32 bits kept after every step (a product that wraps past 2^63 keeps its low bits), so
    the values equal the numpy form's."""
    import torch
    nr, nc = rows.numel(), cols.numel()
    out = torch.empty((nr, nc), dtype=torch.bfloat16, device=rows.device)
    cb = min(nc, block)
    rb = max(1, block // cb)
    for r0 in range(0, nr, rb):
        i = rows[r0:r0 + rb].to(torch.int64).reshape(-1, 1)
        for c0 in range(0, nc, cb):
            j = cols[c0:c0 + cb].to(torch.int64).reshape(1, -1)
            h = (i * _HASH_I + j * _HASH_J + ((seed * _HASH_S) & _MASK32)) & _MASK32
            h ^= h >> 16
            h = (h * 0x7FEB352D) & _MASK32
            h ^= h >> 15
            h = (h * 0x846CA68B) & _MASK32
            h ^= h >> 16
            out[r0:r0 + rb, c0:c0 + cb] = (torch.remainder(h, 2 * span + 1) - span).to(torch.bfloat16)
    return out


def tie_rich(shape, seed: int, dtype: str = "bf16") -> np.ndarray:
    """Values from {-2, -1, -0.0, +0.0, 1, 2, 3}: many equal magnitudes and signed zeros."""
    rng = np.random.Generator(np.random.PCG64(seed))
    alphabet = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, 3.0], np.float32)
    x = alphabet[rng.integers(0, len(alphabet), size=shape)]
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# name -> dict of shapes, distributions and seeds
WORKLOADS = {
    "nm24_fp32_256x512x128": dict(
        kind="spmm_nm", dtype="f32", R=256, K=512, Nc=128,
        A=dict(seed=1000, mean=0.0, std=1.0), B=dict(seed=1001, mean=0.0, std=1.0)),
    "ffn_up_nm24_8192x2048x4096": dict(
        kind="spmm_nm", dtype="bf16", R=8192, K=2048, Nc=4096,
        A=dict(seed=2000, mean=0.0, std=0.02), B=dict(seed=2001, mean=0.0, std=1.0)),
    "ffn_up_nm28_8192x2048x4096": dict(
        kind="spmm_nm_general", dtype="bf16", R=8192, K=2048, Nc=4096, N=2, M=8,
        A=dict(seed=2000, mean=0.0, std=0.02), B=dict(seed=2001, mean=0.0, std=1.0)),
    "ffn_up_nm48_8192x2048x4096": dict(
        kind="spmm_nm_general", dtype="bf16", R=8192, K=2048, Nc=4096, N=4, M=8,
        A=dict(seed=2000, mean=0.0, std=0.02), B=dict(seed=2001, mean=0.0, std=1.0)),
    "ffn_down_vnm64_2_8_2048x8192x4096": dict(
        kind="spmm_venom", dtype="bf16", R=2048, K=8192, Nc=4096, V=64, M=8,
        A=dict(seed=3000, mean=0.0, std=0.02), B=dict(seed=3001, mean=0.0, std=1.0)),
    "train_step_nm24_dmodel4096_dff16384_tok8192": dict(
        kind="train_step", dtype="bf16", d_model=4096, d_ff=16384, tokens=8192,
        W=dict(seed=4000, mean=0.0, std=0.02), X=dict(seed=4001, mean=0.0, std=1.0),
        dY=dict(seed=4002, mean=0.0, std=1.0)),
    "ffn_up_nm24_lowrank64_8192x2048x4096": dict(
        kind="spmm_nm_lowrank", dtype="bf16", R=8192, K=2048, Nc=4096, rank=64,
        A=dict(seed=2000, mean=0.0, std=0.02), B=dict(seed=2001, mean=0.0, std=1.0),
        U=dict(seed=2002, mean=0.0, std=0.02), Vt=dict(seed=2003, mean=0.0, std=0.02)),
    "ffn_block_fwd_nm24_vnm128_dmodel4096_dff16384_tok8192": dict(
        kind="ffn_block", dtype="bf16", d_model=4096, d_ff=16384, tokens=8192, V=128, M=8,
        W=dict(seed=7000, mean=0.0, std=0.02), X=dict(seed=7001, mean=0.0, std=1.0),
        W_down=dict(seed=7002, mean=0.0, std=0.02)),
    "ffn_block_fwd_fused_nm24_vnm128_dmodel4096_dff16384_tok8192": dict(
        kind="ffn_block_fused", dtype="bf16", d_model=4096, d_ff=16384, tokens=8192, V=128, M=8,
        W=dict(seed=7000, mean=0.0, std=0.02), X=dict(seed=7001, mean=0.0, std=1.0),
        W_down=dict(seed=7002, mean=0.0, std=0.02)),
    "relu_act_vnm128_2_8_8192x16384x4096": dict(
        kind="act_venom", dtype="bf16", R=8192, K=16384, Nc=4096, V=128, M=8,
        Z=dict(seed=5000, mean=-0.5, std=1.0), W=dict(seed=5001, mean=0.0, std=0.02)),
    # the backward of the down-projection above: the same activations and weight, and dY [T x Nc]
    "relu_act_vnm128_bwd_8192x16384x4096": dict(
        kind="act_venom_bwd", dtype="bf16", R=8192, K=16384, Nc=4096, V=128, M=8,
        Z=dict(seed=5000, mean=-0.5, std=1.0), W=dict(seed=5001, mean=0.0, std=0.02),
        dY=dict(seed=5002, mean=0.0, std=1.0)),
}
