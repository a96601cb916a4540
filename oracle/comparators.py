"""Comparator row orders for the reordering study, exact integers (test
infrastructure only).

WaveAlign's comparison with other reordering algorithms (Table II) names MinHash
among the alternatives to its spectral Stage 1 without giving its steps; the
method is the published min-wise hashing of sets (Broder), restated here:

* Each query block u is the set S_u of K/V block ids in its mask row.
* Hash functions h_i(v) = (a_i * v + b_i) mod P with P = 2^31 - 1 (a Mersenne
  prime), 1 <= a_i < P and 0 <= b_i < P drawn by the input generator and passed in.
* The signature of u is sig_i(u) = min over v in S_u of h_i(v); an empty row
  takes sig_i = P, above every hash value.  For two rows the probability over the
  hash family that sig_i agrees approximates their Jaccard similarity, so rows with
  equal signatures are likely to share K/V blocks.

Readings (the page leaves how signatures become a row order open):

* The order sorts rows by their signature tuple (sig_1, ..., sig_k)
  lexicographically, ties by row index: rows that share a leading MinHash value,
  which is what an LSH bucket over that value groups, become neighbours.
* The result then goes through the same wave buckets and NNZ-descending Stage 2
  as WaveAlign's own order (reorder.stage2_order), so the comparison isolates the
  spatial ordering.

The LSH comparator (Table II names locality-sensitive hashing; the banded scheme
for min-wise signatures is the standard one, restated here):

* 2B hash functions form B bands of r = 2 signature values each; a row's bucket in
  band b is the exact pair (sig_2b, sig_2b+1), so two rows share it with probability
  about J^2 for Jaccard similarity J, and sharing some bucket among B bands is likely
  only for similar rows.
* Each row joins the lowest-index row it shares a bucket with in any band (itself if
  none is lower): its label.  Reading for the order (the page gives none): rows by
  (label, row), so a group is a row and the higher rows directly similar to it, and
  groups keep the order of their first row.  The relation is not closed
  transitively: on masks whose neighbouring rows overlap strongly, chains of pairs
  would join nearly every row into one group and give back the original order.
  Then the same wave buckets and Stage 2.
"""

from __future__ import annotations

import numpy as np

from .reorder import stage2_order, wave_buckets

MINHASH_P = (1 << 31) - 1


def minhash_signatures(mask_h: np.ndarray, hash_a, hash_b) -> np.ndarray:
    """[MB, k] int64 signatures of the rows of one head's mask."""
    m = np.asarray(mask_h).astype(bool)
    mb, nb = m.shape
    v = np.arange(nb, dtype=np.int64)
    k = len(hash_a)
    sig = np.full((mb, k), MINHASH_P, dtype=np.int64)
    for i in range(k):
        h = (int(hash_a[i]) * v + int(hash_b[i])) % MINHASH_P
        for u in range(mb):
            if m[u].any():
                sig[u, i] = h[m[u]].min()
    return sig


def minhash_order_head(mask_h: np.ndarray, hash_a, hash_b, wave: int, n_slices: int,
                       stage2: bool = True) -> np.ndarray:
    """Execution order of one head: rows by signature, then Stage 2 inside buckets."""
    sig = minhash_signatures(mask_h, hash_a, hash_b)
    mb = sig.shape[0]
    keys = [sig[:, i] for i in range(sig.shape[1] - 1, -1, -1)]
    order = np.lexsort([np.arange(mb)] + keys)  # last key is primary: sig_1, then sig_2, ..., row
    if not stage2:
        return order.astype(np.int64)
    nnz = np.asarray(mask_h).astype(bool).sum(axis=1)
    return stage2_order(order, nnz, wave_buckets(mb, n_slices, wave))


def minhash_order(mask: np.ndarray, hash_a, hash_b, wave: int, n_slices: int,
                  stage2: bool = True):
    """(perm, inv_perm) [H, MB] for every head."""
    H, mb, _ = mask.shape
    perm = np.stack([minhash_order_head(mask[h], hash_a, hash_b, wave, n_slices, stage2)
                     for h in range(H)])
    inv = np.empty_like(perm)
    for h in range(H):
        inv[h, perm[h]] = np.arange(mb)
    return perm, inv


LSH_ROWS_PER_BAND = 2


def lsh_components(mask_h: np.ndarray, hash_a, hash_b, n_bands: int) -> np.ndarray:
    """[MB] label of every row: the lowest row that shares a band bucket with it."""
    k = LSH_ROWS_PER_BAND * n_bands
    sig = minhash_signatures(mask_h, list(hash_a)[:k], list(hash_b)[:k])
    mb = sig.shape[0]
    label = np.arange(mb, dtype=np.int64)
    for b in range(n_bands):
        lowest = {}
        for u in range(mb):  # rows in index order: the first row of a bucket is its lowest
            bucket = (int(sig[u, 2 * b]), int(sig[u, 2 * b + 1]))
            lowest.setdefault(bucket, u)
            label[u] = min(label[u], lowest[bucket])
    return label


def lsh_order_head(mask_h: np.ndarray, hash_a, hash_b, n_bands: int, wave: int, n_slices: int,
                   stage2: bool = True) -> np.ndarray:
    """Execution order of one head: rows by (LSH label, row), then Stage 2."""
    label = lsh_components(mask_h, hash_a, hash_b, n_bands)
    mb = label.size
    order = np.lexsort((np.arange(mb), label))  # by label, then row
    if not stage2:
        return order.astype(np.int64)
    nnz = np.asarray(mask_h).astype(bool).sum(axis=1)
    return stage2_order(order, nnz, wave_buckets(mb, n_slices, wave))


def lsh_order(mask: np.ndarray, hash_a, hash_b, n_bands: int, wave: int, n_slices: int,
              stage2: bool = True):
    """(perm, inv_perm) [H, MB] for every head."""
    H, mb, _ = mask.shape
    perm = np.stack([lsh_order_head(mask[h], hash_a, hash_b, n_bands, wave, n_slices, stage2)
                     for h in range(H)])
    inv = np.empty_like(perm)
    for h in range(H):
        inv[h, perm[h]] = np.arange(mb)
    return perm, inv
