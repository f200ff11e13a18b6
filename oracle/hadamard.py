"""Random-sign Hadamard rotation for FP8 incoherent processing (test infrastructure only).

Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8",
section "Incoherent processing: rotate away the outliers": Q and K are both
multiplied by the orthogonal matrix M = (1/sqrt(d)) H D, where H is the
d x d Sylvester Hadamard matrix and D a random diagonal of +-1 signs. Since
M M^T = I, (Q M)(K M)^T = Q K^T, so the scores are unchanged while an outlier
in one coordinate is spread over all d of them.

The oracle applies M as a dense float64 matrix product (no fast transform):
x -> (x @ H_n) * signs, with H_n = H / sqrt(d) the orthonormal Sylvester
matrix, built by the doubling rule H_{2n} = [[H_n, H_n], [H_n, -H_n]] written
as a Kronecker product.
"""

from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int, normalized: bool = True) -> np.ndarray:
    """n x n Sylvester Hadamard matrix (n a power of two), orthonormal if ``normalized``."""
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Hadamard order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.float64)
    base = np.array([[1.0, 1.0], [1.0, -1.0]])
    while h.shape[0] < n:
        h = np.kron(base, h)
    return h / np.sqrt(n) if normalized else h


def incoherent_rotate(x, signs) -> np.ndarray:
    """Rotate the last axis of x by M = (1/sqrt(d)) H diag(signs): returns x @ M in float64."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    if s.shape != (d,):
        raise ValueError("signs must have one entry per head-dim coordinate")
    return (x @ sylvester_hadamard(d)) * s
