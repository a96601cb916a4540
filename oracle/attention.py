"""Block-masked softmax attention, fp64 (test infrastructure only).

Definition (GSRS §3: attention softmax(QK^T/sqrt(d))V, the block-sparse variant
that excludes unselected blocks from the softmax, and the row-wise LSE that
FlashAttention keeps; WaveAlign §II-C: query block i attends to exactly the
K/V blocks selected by mask row i):

    allowed keys of token row i:  J_i = { j < L : M[i // b, j // b] = 1 }
    z_ij   = s * <q_i, k_j>
    LSE_i  = log sum_{j in J_i} exp(z_ij)          (natural log)
    O_i    = sum_{j in J_i} exp(z_ij - LSE_i) v_j

A row with no allowed key returns O_i = 0 and LSE_i = -inf (GSRS, note on fully
masked rows to Algorithm 2).  Keys j >= L (block padding) are never allowed.
Query rows i >= L are padding: they are not part of the result and come back
as NaN so that no test can compare them by accident.
"""

from __future__ import annotations

import numpy as np


def _keys_of_row(mask_row: np.ndarray, seq_len: int, block: int) -> np.ndarray:
    blocks = np.flatnonzero(mask_row)
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    keys = [np.arange(v * block, min((v + 1) * block, seq_len)) for v in blocks]
    return np.concatenate(keys)


def masked_attention_rows(q_h: np.ndarray, k_h: np.ndarray, v_h: np.ndarray,
                          mask_h: np.ndarray, rows: np.ndarray, seq_len: int,
                          block: int, scale: float):
    """O and LSE for the given token rows of one head (all rows must be < L)."""
    rows = np.asarray(rows, dtype=np.int64)
    d = v_h.shape[1]
    out = np.zeros((rows.size, d), dtype=np.float64)
    lse = np.full(rows.size, -np.inf, dtype=np.float64)
    qb = rows // block
    for u in np.unique(qb):
        sel = np.flatnonzero(qb == u)
        keys = _keys_of_row(mask_h[u], seq_len, block)
        if keys.size == 0:
            continue  # O = 0, LSE = -inf
        z = scale * (q_h[rows[sel]] @ k_h[keys].T)
        m = z.max(axis=1)
        row_lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
        lse[sel] = row_lse
        out[sel] = np.exp(z - row_lse[:, None]) @ v_h[keys]
    return out, lse


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     seq_len: int, block: int, scale: float):
    """O [H, L_pad, d] and LSE [H, L_pad] for every head; padding rows are NaN."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    H, lp, d = q.shape
    out = np.full((H, lp, d), np.nan)
    lse = np.full((H, lp), np.nan)
    rows = np.arange(seq_len)
    for h in range(H):
        o_h, l_h = masked_attention_rows(q[h], k[h], v[h], mask[h], rows, seq_len, block, scale)
        out[h, :seq_len] = o_h
        lse[h, :seq_len] = l_h
    return out, lse


def attention_entropy(q: np.ndarray, k: np.ndarray, mask: np.ndarray, seq_len: int, block: int,
                      scale: float) -> np.ndarray:
    """Entropy of each row's masked attention, -sum_j A_ij ln A_ij (GSRS §4, Fig. 1),
    [H, L_pad]; 0 for a row with no allowed key, NaN on padding rows."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    H, lp, _ = q.shape
    out = np.full((H, lp), np.nan)
    for h in range(H):
        for u in range(lp // block):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            if r1 <= r0:
                continue
            keys = _keys_of_row(mask[h, u], seq_len, block)
            if keys.size == 0:
                out[h, r0:r1] = 0.0
                continue
            z = scale * (q[h, r0:r1] @ k[h, keys].T)
            z = z - z.max(axis=1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=1, keepdims=True)
            with np.errstate(divide="ignore", invalid="ignore"):
                terms = np.where(a > 0, a * np.log(a), 0.0)
            out[h, r0:r1] = -terms.sum(axis=1)
    return out


def attention_distance(q: np.ndarray, k: np.ndarray, mask: np.ndarray, seq_len: int, block: int,
                       scale: float) -> np.ndarray:
    """Mean attention distance of each row, D(i) = sum_j A_ij |i - j| over the row's
    allowed keys, with i and j token positions in the stored sequence order (GSRS §4,
    Fig. 1, and the appendix on fused attention statistics), [H, L_pad]; 0 for a row
    with no allowed key, NaN on padding rows."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    H, lp, _ = q.shape
    out = np.full((H, lp), np.nan)
    for h in range(H):
        for u in range(lp // block):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            if r1 <= r0:
                continue
            keys = _keys_of_row(mask[h, u], seq_len, block)
            if keys.size == 0:
                out[h, r0:r1] = 0.0
                continue
            z = scale * (q[h, r0:r1] @ k[h, keys].T)
            z = z - z.max(axis=1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=1, keepdims=True)
            dist = np.abs(np.arange(r0, r1)[:, None] - keys[None, :]).astype(np.float64)
            out[h, r0:r1] = (a * dist).sum(axis=1)
    return out
