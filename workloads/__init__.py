"""Seeded synthetic inputs for the MRU prefix-scan path.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark.  It holds shapes, noise scales, seeds and random draws only: no step
of the method (no LDU fill, no product, no scan) lives here, so that neither
side of a parity comparison can borrow arithmetic from the other.

Input recipe (one raw parameter vector x_t per token and head):

* ``x`` has shape ``[B, H, T, n*n]`` and dtype float32.  Viewed row-major as an
  n-by-n matrix X_t, its diagonal entries are drawn N(0, sigma_diag) and its
  off-diagonal entries N(0, sigma_off), where N(0, s) means standard
  deviation s.  (The MRU pages describe filling LDU factors from the token
  vector, "Improving Matrix Recurrent Units as an Attention Alternative",
  Key Points; the workload table fixes the scales.)
* Every (b, h) sequence has its own PCG64 stream seeded with
  ``SeedSequence([seed, b, h])``; standard normals are drawn in float64 with
  shape ``[T, n, n]``, scaled, then rounded to float32 (round to nearest even).
  Because the stream is per sequence and sequential, the first t tokens of a
  sequence do not depend on T, so prefixes and subsets of (b, h) can be
  regenerated cheaply.
* Upstream gradients ``R = dL/dP`` are N(0, 1) float32 with shape
  ``[B, H, T, n, n]`` from ``SeedSequence([seed, b, h, 1])``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "gen_x", "gen_R", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    n: int
    sigma_off: float
    sigma_diag: float
    seed: int
    backward: bool = False
    note: str = ""

    @property
    def S(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 1024, 4, 0.1, 0.05, 1,
                   note="small forward-only case, one sequence of 1024 tokens"),
    "c2": Workload("c2", 8, 8, 256, 8, 0.1, 0.05, 2,
                   note="char-LM shaped: d_model 512 = 8 heads x 8x8"),
    "c2l": Workload("c2l", 1024, 8, 256, 8, 0.1, 0.05, 2,
                    note="char-LM shaped with batch 1024 (first 8 batch rows equal c2)"),
    "c3": Workload("c3", 4, 16, 8192, 16, 0.05, 0.02, 3,
                   note="n=16, long sequences"),
    "c4": Workload("c4", 1, 8, 65536, 32, 0.02, 0.01, 4,
                   note="n=32, long context"),
    "c5": Workload("c5", 8, 8, 4096, 16, 0.05, 0.02, 5, backward=True,
                   note="n=16 forward and backward"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _seq_rng(seed: int, b: int, h: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, h, *extra])))


def gen_x(B: int, H: int, T: int, n: int, sigma_off: float, sigma_diag: float, seed: int,
          b_idx=None, h_idx=None) -> np.ndarray:
    """Raw per-token parameter vectors, ``[len(b_idx), len(h_idx), T, n*n]`` float32.

    ``b_idx``/``h_idx`` select a subset of sequences (default: all); a selected
    sequence gets exactly the values it has in the full tensor.
    """
    bs = range(B) if b_idx is None else list(b_idx)
    hs = range(H) if h_idx is None else list(h_idx)
    out = np.empty((len(bs), len(hs), T, n * n), dtype=np.float32)
    scale = np.full((n, n), float(sigma_off))
    np.fill_diagonal(scale, float(sigma_diag))
    for i, b in enumerate(bs):
        for j, h in enumerate(hs):
            z = _seq_rng(seed, b, h).standard_normal((T, n, n))
            out[i, j] = (z * scale).astype(np.float32).reshape(T, n * n)
    return out


def gen_R(B: int, H: int, T: int, n: int, seed: int, b_idx=None, h_idx=None) -> np.ndarray:
    """Upstream gradient dL/dP, ``[len(b_idx), len(h_idx), T, n, n]`` float32, N(0, 1)."""
    bs = range(B) if b_idx is None else list(b_idx)
    hs = range(H) if h_idx is None else list(h_idx)
    out = np.empty((len(bs), len(hs), T, n, n), dtype=np.float32)
    for i, b in enumerate(bs):
        for j, h in enumerate(hs):
            out[i, j] = _seq_rng(seed, b, h, 1).standard_normal((T, n, n)).astype(np.float32)
    return out


def gen_for(w: Workload, T: int | None = None, b_idx=None, h_idx=None):
    """Convenience: (x, R-or-None) for a workload, optionally truncated to T tokens."""
    T = w.T if T is None else T
    x = gen_x(w.B, w.H, T, w.n, w.sigma_off, w.sigma_diag, w.seed, b_idx, h_idx)
    R = gen_R(w.B, w.H, T, w.n, w.seed, b_idx, h_idx) if w.backward else None
    return x, R
