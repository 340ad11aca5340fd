"""Gradual magnitude pruning driver over the library's N:M calls.

"Success story: ESPLAG" (Highlights, Research Topic) co-designs the sparse
kernels with a semi-structured gradual magnitude pruning technique; "To 2:4
Sparsity and Beyond" (abstract) trains with sparse steps and switches to regular
dense steps towards the end.  The schedule itself -- which N:M pattern holds at
which step -- is the library's host function `nm_gmp_n_at` (its header states
the ramp); this module only sequences the library's calls around the caller's
training steps:

  * before the ramp and after the dense switch the weight is used densely;
  * at a pruning event the current weight is magnitude-pruned to the event's
    N:M (nm_prune_compress), and the pruned entries of the dense master weight
    are set to +0.0 (nm_decompress of the compressed form), so a later event --
    a sparser pattern -- keeps them pruned;
  * between events the mask is held: the caller updates the kept entries of the
    master weight, and each step recompresses it under that mask (nm_compress).

Every step of the computation runs in the library's kernels; nothing here
computes on tensors.
"""

from __future__ import annotations

import ctypes

import torch

from . import nmsparse as _nm


class GradualPruner:
    """Holds the master weight W [R, K] (device, bf16 or fp32; updated in place by the caller)
    and its current compressed form.  Call step(t) at the start of training step t."""

    def __init__(self, W: torch.Tensor, M: int, n_final: int, t_begin: int, t_end: int, interval: int,
                 t_dense: int = -1):
        if W.dim() != 2 or not W.is_cuda:
            raise ValueError("W must be a 2-D device tensor")
        self.W, self.M = W, M
        self.params = (M, n_final, t_begin, t_end, interval, t_dense)
        if self.schedule(0)[0] < 0:
            raise ValueError("invalid schedule parameters")
        self.N = M
        self.mask = self.values = self.meta = None

    def schedule(self, step: int):
        """(N in effect at `step` (M when dense), whether `step` is a pruning event)."""
        prune = ctypes.c_int(0)
        n = _nm.lib().nm_gmp_n_at(*self.params, step, ctypes.byref(prune))
        return n, bool(prune.value)

    @property
    def sparse(self) -> bool:
        return self.values is not None

    def step(self, t: int) -> int:
        """Bring the weight's form up to date for step t; returns the N in effect (M: dense)."""
        N, prune = self.schedule(t)
        R, K = self.W.shape
        if N == self.M:
            # dense: before the ramp, or the switch to dense steps (the master weight already holds
            # zeros at the pruned entries; from now on every entry is trained)
            self.N, self.mask, self.values, self.meta = N, None, None, None
            return N
        if prune:
            self.mask, self.values, self.meta = _nm.nm_prune_compress(self.W, N, self.M)
            _nm.nm_decompress(self.values, self.meta, K, N, self.M, out=self.W)
            self.N = N
        else:
            self.values, self.meta = _nm.nm_compress(self.W, self.mask, self.N, self.M, values=self.values,
                                                     meta=self.meta)
        return self.N
