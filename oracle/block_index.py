"""Compressed block index of a block mask (test infrastructure only).

WaveAlign §II-B/§II-C: mask row i lists the K/V blocks that query block i
visits in the kernel's inner loop, and its row sum n_i = sum_j M_ij (the NNZ)
is that query block's workload.  The index is the plain definition written
out: for each head h and row u (head-major order), the ascending list of v with
M[h, u, v] = 1; ``row_ptr`` is the exclusive prefix sum of the row counts over
all H*MB rows.  The column index (CSC) is the same for the transposed mask,
with ``csc_ptr`` over all H*NB columns and row ids local to the head.
"""

from __future__ import annotations

import numpy as np


def block_index(mask: np.ndarray):
    """Return (row_ptr, col_idx, row_nnz, csc_ptr, csc_idx) as int64 arrays."""
    mask = np.asarray(mask)
    H, MB, NB = mask.shape
    row_nnz = np.zeros(H * MB, dtype=np.int64)
    cols = []
    for h in range(H):
        for u in range(MB):
            nz = np.flatnonzero(mask[h, u])
            row_nnz[h * MB + u] = nz.size
            cols.append(nz)
    row_ptr = np.zeros(H * MB + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(row_nnz)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
    csc_cnt = np.zeros(H * NB, dtype=np.int64)
    rows = []
    for h in range(H):
        for v in range(NB):
            nz = np.flatnonzero(mask[h, :, v])
            csc_cnt[h * NB + v] = nz.size
            rows.append(nz)
    csc_ptr = np.zeros(H * NB + 1, dtype=np.int64)
    csc_ptr[1:] = np.cumsum(csc_cnt)
    csc_idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return row_ptr, col_idx.astype(np.int64), row_nnz, csc_ptr, csc_idx.astype(np.int64)
