"""GSRS fused block importance and Top-p selection, fp64 (test infrastructure only).

Restates "Sparse Attention for Video Generation Acceleration via Growing
Sparsity and Reduced Search" (GSRS).  The page's display equations were lost in
extraction; the readings below follow its prose:

* Phase 1 (§5.3, Appendix A.2): for query row i and evaluated key block v,
  G_iv = m_iv + log r_iv with m_iv the block maximum of z_ij over the valid keys
  of v and r_iv = sum_j exp(z_ij - m_iv); this is the block log-sum-exp.  A block
  without valid keys gives -inf.
* Row normaliser: L_i = log sum over all evaluated keys of exp(z_ij).
* Phase 2: W_uv = (1 / B_u) sum over the valid rows i of query block u of
  exp(G_iv - L_i), B_u the number of valid rows; rows with L_i = -inf add 0
  (note on fully masked rows to Algorithm 2).  Hence sum_v W_uv = 1.
* Top-p (Algorithm 3, "retained until their cumulative importance exceeds a
  threshold p"): candidates of a row sorted by descending W (equal W: lower
  block id first); the running total is accumulated in fp64 in that order and a
  block is kept while the total *before* it is <= p, so the block whose
  addition first takes the total above p is the last one kept.
"""

from __future__ import annotations

import numpy as np


def _valid_keys(v: int, seq_len: int, block: int) -> np.ndarray:
    return np.arange(v * block, min((v + 1) * block, seq_len))


def block_lse(q: np.ndarray, k: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray,
              seq_len: int, block: int, scale: float):
    """Phase 1: G [nnz, block] (CSR order) and the row LSE [H, L_pad] over the evaluated keys.

    Query rows >= L are NaN in both outputs.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    H, lp, _ = q.shape
    mb = lp // block
    nnz = int(row_ptr[-1])
    g = np.full((nnz, block), np.nan)
    lse = np.full((H, lp), np.nan)
    for h in range(H):
        for u in range(mb):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            if r1 <= r0:
                continue
            lo, hi = int(row_ptr[h * mb + u]), int(row_ptr[h * mb + u + 1])
            if hi == lo:
                lse[h, r0:r1] = -np.inf
                continue
            qs = q[h, r0:r1]
            allz = []
            for e in range(lo, hi):
                keys = _valid_keys(int(col_idx[e]), seq_len, block)
                z = scale * (qs @ k[h, keys].T)
                allz.append(z)
                if keys.size == 0:
                    g[e, : r1 - r0] = -np.inf
                    continue
                m = z.max(axis=1)
                g[e, : r1 - r0] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
            z = np.concatenate(allz, axis=1)
            m = z.max(axis=1)
            lse[h, r0:r1] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return g, lse


def block_importance(g: np.ndarray, lse: np.ndarray, row_ptr: np.ndarray, seq_len: int,
                     block: int) -> np.ndarray:
    """Phase 2: W [nnz] from G and the row LSE."""
    H, lp = lse.shape
    mb = lp // block
    w = np.zeros(g.shape[0])
    for h in range(H):
        for u in range(mb):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            nrows = r1 - r0
            if nrows <= 0:
                continue
            l_rows = np.asarray(lse[h, r0:r1], dtype=np.float64)
            live = np.isfinite(l_rows)
            for e in range(int(row_ptr[h * mb + u]), int(row_ptr[h * mb + u + 1])):
                gi = np.asarray(g[e, :nrows], dtype=np.float64)
                terms = np.where(live, np.exp(np.where(live, gi - l_rows, 0.0)), 0.0)
                terms = np.where(np.isneginf(gi), 0.0, terms)
                w[e] = terms.sum() / nrows
    return w


def block_importance_from_probs(q: np.ndarray, k: np.ndarray, row_ptr: np.ndarray,
                                col_idx: np.ndarray, seq_len: int, block: int,
                                scale: float) -> np.ndarray:
    """W from explicit attention probabilities A_ij = exp(z_ij - L_i) (GSRS eq. (5)).

    The block importance as defined: the attention weight of row i on the keys
    of block v, normalised over the evaluated keys, averaged over the rows of u.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    H, lp, _ = q.shape
    mb = lp // block
    w = np.zeros(int(row_ptr[-1]))
    for h in range(H):
        for u in range(mb):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            lo, hi = int(row_ptr[h * mb + u]), int(row_ptr[h * mb + u + 1])
            if r1 <= r0 or hi == lo:
                continue
            blocks = [int(col_idx[e]) for e in range(lo, hi)]
            keys = np.concatenate([_valid_keys(v, seq_len, block) for v in blocks])
            z = scale * (q[h, r0:r1] @ k[h, keys].T)
            z = z - z.max(axis=1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=1, keepdims=True)
            col = 0
            for e, v in zip(range(lo, hi), blocks):
                n = _valid_keys(v, seq_len, block).size
                w[e] = a[:, col:col + n].sum() / (r1 - r0)
                col += n
    return w


def cached_lse_scores(g: np.ndarray, lse_old: np.ndarray, row_ptr: np.ndarray,
                      seq_len: int, block: int) -> np.ndarray:
    """Per-row block scores exp(G_iv - L_i^old) with a stale row normaliser.

    GSRS Appendix (AdaSpa comparison): these sum to exp(L_i - L_i^old) per row,
    not to 1.  Returned as [nnz, block] (NaN on padding rows).
    """
    H, lp = lse_old.shape
    mb = lp // block
    s = np.full(g.shape, np.nan)
    for h in range(H):
        for u in range(mb):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            for e in range(int(row_ptr[h * mb + u]), int(row_ptr[h * mb + u + 1])):
                s[e, : r1 - r0] = np.exp(g[e, : r1 - r0] - lse_old[h, r0:r1])
    return s


def topp_select(w: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray, heads: int,
                mb: int, nb: int, p: float) -> np.ndarray:
    """GSRS Algorithm 3 per query-block row: mask [H, MB, NB] of the kept blocks."""
    out = np.zeros((heads, mb, nb), dtype=np.uint8)
    w = np.asarray(w)
    for h in range(heads):
        for u in range(mb):
            lo, hi = int(row_ptr[h * mb + u]), int(row_ptr[h * mb + u + 1])
            if hi == lo:
                continue
            cand = np.asarray(col_idx[lo:hi], dtype=np.int64)
            ww = w[lo:hi].astype(np.float64)
            order = np.lexsort((cand, -ww))  # by -W, then by block id
            acc = 0.0
            for j in order:
                if acc > p:
                    break
                out[h, u, cand[j]] = 1
                acc += float(ww[j])
    return out


def mask_recall(q: np.ndarray, k: np.ndarray, mask: np.ndarray, seq_len: int, block: int,
                scale: float) -> np.ndarray:
    """GSRS §3 attention recall of a block mask, per query block [H, MB].

    The share of the full attention A = softmax(scale * q k^T) (over all keys below
    seq_len) that falls on the key blocks the mask keeps, averaged over the valid
    rows of each query block.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    H, lp, _ = q.shape
    mb = lp // block
    out = np.zeros((H, mb))
    for h in range(H):
        z = scale * (q[h, :seq_len] @ k[h, :seq_len].T)
        z = z - z.max(axis=1, keepdims=True)
        a = np.exp(z)
        a = a / a.sum(axis=1, keepdims=True)
        for u in range(mb):
            r0, r1 = u * block, min((u + 1) * block, seq_len)
            kept = [v for v in range(mb) if mask[h, u, v]]
            if r1 <= r0 or not kept:
                continue
            keys = np.concatenate([_valid_keys(v, seq_len, block) for v in kept])
            out[h, u] = a[r0:r1][:, keys].sum() / (r1 - r0)
    return out


def gsrs_schedule(steps: int, search_steps, thresholds, qk_at, seq_len: int, block: int,
                  scale: float, w_select=None):
    """The GSRS inference schedule over denoising steps (GSRS §4-5: warmup, growing
    sparsity, reduced search, mask reuse; Algorithm 4 is named there and its
    control flow described in the prose), as a plain loop.

    Reading of the schedule (T = search_steps, p = thresholds):

    * t < T[0]: warmup, dense attention (every block kept);
    * t = T[0]: first search over all blocks: Phase-1 G and row LSE of the dense
      pass, W (Phase 2), Top-p at p[0]; the kept set is the candidate set S1 and
      the current mask;
    * t = T[k], k >= 1: reduced search inside S1: G and LSE of the pass over S1,
      W normalised over S1, Top-p at p[k]; the kept set (inside S1) is the current
      mask;
    * any other t > T[0]: the current mask is reused.

    ``qk_at(t)`` gives the (q, k) arrays [H, L_pad, d] of step t.  ``w_select`` maps a
    search step to the block weights (CSR order of that search's candidate set) that
    its Top-p runs on; by default the oracle's own W.  Returns (kinds, masks, weights):
    the kind of every step, the mask [H, MB, NB] every step runs with, and the
    oracle's W at every search step.
    """
    T, p = tuple(search_steps), tuple(thresholds)
    if len(T) != len(p) or list(T) != sorted(T) or T[-1] >= steps:
        raise ValueError("one threshold per increasing search step below the step count")
    w_select = w_select or {}
    kinds, masks, weights = [], [], {}
    s1 = mask = dense = None
    for t in range(steps):
        q, k = qk_at(t)
        if dense is None:
            H, lp, _ = q.shape
            mb = lp // block
            dense = np.ones((H, mb, mb), dtype=np.uint8)
        if t < T[0]:
            kinds.append("warmup")
            masks.append(dense)
            continue
        if t in T:
            cand = dense if t == T[0] else s1
            rp, ci, _, _, _ = block_index_of(cand)
            g, lse = block_lse(q, k, rp, ci, seq_len, block, scale)
            w = block_importance(g, lse, rp, seq_len, block)
            weights[t] = w
            w_used = w_select.get(t, w)
            kept = topp_select(w_used, rp, ci, cand.shape[0], cand.shape[1], cand.shape[2],
                               p[T.index(t)])
            if t == T[0]:
                s1 = kept
            mask = kept
            kinds.append("search")
        else:
            kinds.append("reuse")
        masks.append(mask)
    return kinds, masks, weights


def block_index_of(mask: np.ndarray):
    """The CSR of a block mask (the oracle's block_index, imported lazily)."""
    from .block_index import block_index
    return block_index(mask)
