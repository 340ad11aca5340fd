"""The counter-based integer generator of the synthetic inputs: its numpy and torch forms give the
same entries (any block regenerated alone equals the same block of a larger draw), within
[-span, span], every value drawn."""

import numpy as np
import torch

from sparse_matmul_ffns_amd import synth


def test_hashed_ints_numpy_and_torch_agree():
    rows = np.array([0, 1, 2, 3, 4095, 524287, 524288, 2**20 - 1, 2**20 + 255, 2**23 - 1])
    cols = np.arange(0, 8192, 13)
    for seed, span in ((0, 3), (42, 1), (7, 8)):
        a = synth.hashed_ints(rows, cols, seed, span)
        b = synth.hashed_ints_torch(torch.tensor(rows), torch.tensor(cols), seed, span, block=1000)
        assert np.array_equal(a, b.view(torch.int16).numpy().view(np.uint16))
        v = synth.bf16_bits_to_f32(a)
        assert v.min() >= -span and v.max() <= span and np.all(v == np.round(v))
        assert len(np.unique(v)) == 2 * span + 1


def test_hashed_ints_blocks_regenerate():
    full = synth.hashed_ints(np.arange(64), np.arange(96), 5)
    assert np.array_equal(full[10:20, 30:41], synth.hashed_ints(np.arange(10, 20), np.arange(30, 41), 5))
    assert not np.array_equal(full, synth.hashed_ints(np.arange(64), np.arange(96), 6))
    assert not np.array_equal(full[:, :64], full[:, :64].T)
