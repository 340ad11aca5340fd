"""The panel layout of a 2:4 form, written out on the host (a pure reordering of bytes): the
values piece of row r and 64-column step s at line (r // 2) * (K // 64) + s, half r % 2; the
metadata piece of row r and 256-column chunk c at line (r // 4) * (K // 256) + c, quarter r % 4."""

import numpy as np


def values_to_panels(values: np.ndarray, R: int, K: int) -> np.ndarray:
    """values [R][K/2] (any 2-byte dtype) -> the panel layout, flat."""
    v = np.ascontiguousarray(values).reshape(R // 2, 2, K // 64, 32)
    return np.ascontiguousarray(v.transpose(0, 2, 1, 3)).reshape(-1)


def meta_to_panels(meta: np.ndarray, R: int, K: int) -> np.ndarray:
    """meta [R][K/8] bytes -> the panel layout, flat."""
    m = np.ascontiguousarray(meta).reshape(R // 4, 4, K // 256, 32)
    return np.ascontiguousarray(m.transpose(0, 2, 1, 3)).reshape(-1)


def values_from_panels(vp: np.ndarray, R: int, K: int) -> np.ndarray:
    v = np.asarray(vp).reshape(R // 2, K // 64, 2, 32)
    return np.ascontiguousarray(v.transpose(0, 2, 1, 3)).reshape(R, K // 2)


def meta_from_panels(mp: np.ndarray, R: int, K: int) -> np.ndarray:
    m = np.asarray(mp).reshape(R // 4, K // 256, 4, 32)
    return np.ascontiguousarray(m.transpose(0, 2, 1, 3)).reshape(R, K // 8)
