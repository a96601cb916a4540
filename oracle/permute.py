"""Explicit row permutation of block-structured tensors (test infrastructure only).

WaveAlign §V: the reordering operator gathers the query blocks (and mask rows)
into the scheduled order before the kernel, and the inverse operator puts the
output rows back.  With ``perm[h, s]`` the original block run at position s:

    gathered[h, s*b:(s+1)*b] = x[h, perm[h, s]*b:(perm[h, s]+1)*b]
    restored[h, perm[h, s]*b:(perm[h, s]+1)*b] = y[h, s*b:(s+1)*b]
"""

from __future__ import annotations

import numpy as np


def gather_blocks(x: np.ndarray, perm: np.ndarray, rows_per_block: int) -> np.ndarray:
    H, mb = perm.shape
    out = np.empty_like(x)
    for h in range(H):
        for s in range(mb):
            src = perm[h, s] * rows_per_block
            out[h, s * rows_per_block:(s + 1) * rows_per_block] = x[h, src:src + rows_per_block]
    return out


def scatter_blocks(y: np.ndarray, perm: np.ndarray, rows_per_block: int) -> np.ndarray:
    H, mb = perm.shape
    out = np.empty_like(y)
    for h in range(H):
        for s in range(mb):
            dst = perm[h, s] * rows_per_block
            out[h, dst:dst + rows_per_block] = y[h, s * rows_per_block:(s + 1) * rows_per_block]
    return out
