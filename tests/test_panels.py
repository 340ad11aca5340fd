"""The host form of the panel layout (tests/panels.py) against its definition, element by element
(CPU), and the status codes of the three panel-layout calls (no call here reaches a kernel)."""

import numpy as np

from sparse_matmul_ffns_amd import nmsparse as nm
from tests.panels import meta_from_panels, meta_to_panels, values_from_panels, values_to_panels

FAKE = 4096


def test_values_layout_by_definition():
    R, K = 8, 512
    vals = np.arange(R * K // 2, dtype=np.uint16).reshape(R, K // 2)   # value j of row r = r*K/2 + j
    vp = values_to_panels(vals, R, K)
    assert vp.size == vals.size
    for r in range(R):
        for s in range(K // 64):
            base = ((r // 2) * (K // 64) + s) * 64 + (r % 2) * 32     # in 2-byte elements
            assert np.array_equal(vp[base:base + 32], vals[r, 32 * s:32 * s + 32])
    assert np.array_equal(values_from_panels(vp, R, K), vals)


def test_meta_layout_by_definition():
    R, K = 12, 768
    meta = (np.arange(R * K // 8) % 251).astype(np.uint8).reshape(R, K // 8)
    mp = meta_to_panels(meta, R, K)
    for r in range(R):
        for c in range(K // 256):
            base = ((r // 4) * (K // 256) + c) * 128 + (r % 4) * 32
            assert np.array_equal(mp[base:base + 32], meta[r, 32 * c:32 * c + 32])
    assert np.array_equal(meta_from_panels(mp, R, K), meta)


def test_panel_call_errors():
    L, s = nm.lib(), None
    # nm_to_panels(dt, values, meta, R, K, values_p, meta_p, stream)
    assert L.nm_to_panels(1, FAKE, None, 4, 256, FAKE, FAKE, s) == nm.NM_ERR_NULL
    assert L.nm_to_panels(0, FAKE, FAKE, 4, 256, FAKE, FAKE, s) == nm.NM_ERR_UNSUPPORTED
    assert L.nm_to_panels(1, FAKE, FAKE, 6, 256, FAKE, FAKE, s) == nm.NM_ERR_SHAPE
    assert L.nm_to_panels(1, FAKE, FAKE, 4, 128, FAKE, FAKE, s) == nm.NM_ERR_SHAPE
    assert L.nm_to_panels(1, FAKE, FAKE + 8, 4, 256, FAKE, FAKE, s) == nm.NM_ERR_ALIGN
    # nm_reprune_t_transpose_panels(dt, values, meta, R, K, values_t, meta_t, X, ldx, RX, CX, Xt, ldxt, stream)
    args = [FAKE, FAKE, 256, 128, FAKE, FAKE, FAKE, 8, 8, 8, FAKE, 8, s]
    assert L.nm_reprune_t_transpose_panels(0, *args) == nm.NM_ERR_UNSUPPORTED
    bad = list(args); bad[2] = 128                       # R not a multiple of 256
    assert L.nm_reprune_t_transpose_panels(1, *bad) == nm.NM_ERR_SHAPE
    bad = list(args); bad[3] = 64                        # K not a multiple of 128
    assert L.nm_reprune_t_transpose_panels(1, *bad) == nm.NM_ERR_SHAPE
    bad = list(args); bad[7] = 4                         # ldx < CX
    assert L.nm_reprune_t_transpose_panels(1, *bad) == nm.NM_ERR_SHAPE
    bad = list(args); bad[4] = FAKE + 2                  # values_t not 16-byte aligned
    assert L.nm_reprune_t_transpose_panels(1, *bad) == nm.NM_ERR_ALIGN
    bad = list(args); bad[6] = None
    assert L.nm_reprune_t_transpose_panels(1, *bad) == nm.NM_ERR_NULL
    # spmm_nm_t_panels(dt, values, meta, R, K, Bt, ldbt, Nc, C, ldc, stream)
    args = [FAKE, FAKE, 256, 256, FAKE, 256, 8, FAKE, 8, s]
    assert L.spmm_nm_t_panels(0, *args) == nm.NM_ERR_UNSUPPORTED
    for i, v in ((2, 128), (3, 128), (5, 200), (5, 260), (8, 4)):
        bad = list(args); bad[i] = v
        assert L.spmm_nm_t_panels(1, *bad) == nm.NM_ERR_SHAPE, (i, v)
    bad = list(args); bad[1] = FAKE + 4
    assert L.spmm_nm_t_panels(1, *bad) == nm.NM_ERR_ALIGN
    bad = list(args); bad[7] = FAKE + 2
    assert L.spmm_nm_t_panels(1, *bad) == nm.NM_ERR_ALIGN
    bad = list(args); bad[0] = None
    assert L.spmm_nm_t_panels(1, *bad) == nm.NM_ERR_NULL
    bad = list(args); bad[2], bad[3], bad[5] = 1 << 16, 1 << 16, 1 << 16   # values of 4 GiB
    assert L.spmm_nm_t_panels(1, *bad) == nm.NM_ERR_TOO_LARGE
