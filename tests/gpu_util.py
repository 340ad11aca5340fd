"""Helpers for the GPU parity tests: move raw bit arrays to and from the device."""

import numpy as np
import pytest
import torch

from oracle import nm_oracle as O


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev(raw: np.ndarray, dtype: str, pad: int = 0) -> torch.Tensor:
    """numpy raw array -> device tensor (bf16 from its bit patterns); `pad` extra
    columns make the row stride larger than the width (a strided view is returned)."""
    if raw.ndim == 2 and pad:
        wide = np.zeros((raw.shape[0], raw.shape[1] + pad), raw.dtype)
        wide[:, :raw.shape[1]] = raw
        return dev(wide, dtype)[:, :raw.shape[1]]
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16).copy()).view(torch.bfloat16).cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw).copy()).cuda()
    if dtype == "u8":
        return torch.from_numpy(np.ascontiguousarray(raw).copy()).cuda()
    raise ValueError(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy raw array (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_close(C_gpu: np.ndarray, C_ref: np.ndarray, bound: np.ndarray, what: str):
    """The floating-point acceptance test: relative Frobenius <= 1e-3 and
    |C - C*| <= 1e-2 * (|A| |B|) elementwise, against the fp64 oracle."""
    ok, fro, worst = O.within_tolerance(C_gpu, C_ref, bound)
    assert ok, f"{what}: rel Frobenius {fro:.3e}, worst elementwise excess {worst:.3e}"
    return fro
