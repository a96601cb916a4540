"""Cache-locality proxies of a query-block execution order, on the host (NumPy).

They rate an order before (or beside) GPU counters.  A head's order is cut, as the
XCD-sliced schedule runs it, into ``n_slices`` contiguous slices (one per XCD) and
each slice into waves of ``wave`` positions (the workgroups resident on one XCD at
once).

* ``wave_objective``: WaveAlign's Problem (1) (§IV-B, eq. (1)): the sum over the
  waves of the squared distances between every two mask rows of the wave,
  sum_{i,j in wave} ||M_i - M_j||^2 = 2 R sum_i n_i - 2 ||sum_i M_i||^2 for binary
  rows (R rows, n_i = |M_i|).  Lower is better.
* ``distinct_kv_per_wave``: the mean number of distinct K/V blocks a wave needs.
* ``lru_l2_model``: a model of one XCD's L2 serving the K/V tiles: each XCD runs its
  slices head after head on ``slots`` workgroup slots with greedy list scheduling
  (a free slot takes the next query block of the slice), a query block visits one
  K/V tile per time step in ascending block order, and the L2 keeps the
  ``lru_tiles`` most recently used tiles (4 MB / 64 KB = 64 on MI355X).  Returns
  the modelled hit rate of the tile accesses.
"""

from __future__ import annotations

from collections import OrderedDict

import numpy as np


def _waves(mb: int, n_slices: int, wave: int):
    s = -(-mb // n_slices)
    for x in range(n_slices):
        lo, hi = x * s, min((x + 1) * s, mb)
        for b in range(lo, hi, wave):
            yield x, b, min(b + wave, hi)


def wave_objective(mask: np.ndarray, perm: np.ndarray, n_slices: int, wave: int) -> float:
    """Problem (1) summed over all heads and waves of the order ``perm`` [H, MB]."""
    m = np.asarray(mask).astype(np.int64)
    total = 0
    for h in range(m.shape[0]):
        for _, lo, hi in _waves(m.shape[1], n_slices, wave):
            rows = m[h, perm[h, lo:hi]]
            n = rows.sum()
            col = rows.sum(axis=0)
            total += 2 * (hi - lo) * int(n) - 2 * int((col * col).sum())
    return float(total)


def distinct_kv_per_wave(mask: np.ndarray, perm: np.ndarray, n_slices: int, wave: int) -> float:
    m = np.asarray(mask).astype(bool)
    counts = []
    for h in range(m.shape[0]):
        for _, lo, hi in _waves(m.shape[1], n_slices, wave):
            counts.append(int(m[h, perm[h, lo:hi]].any(axis=0).sum()))
    return float(np.mean(counts)) if counts else 0.0


def lru_l2_model(mask: np.ndarray, perm: np.ndarray, n_slices: int, slots: int,
                 lru_tiles: int, heads=None) -> float:
    """Modelled L2 hit rate of the K/V tile accesses, over the given heads (all by
    default), every XCD with its own L2."""
    m = np.asarray(mask).astype(bool)
    H, mb, _ = m.shape
    heads = range(H) if heads is None else heads
    s = -(-mb // n_slices)
    lists = {}
    hits = accesses = 0
    for x in range(n_slices):
        cache = OrderedDict()
        queue = []
        for h in heads:
            for pos in range(x * s, min((x + 1) * s, mb)):
                queue.append((h, int(perm[h, pos])))
        qi = 0
        active = []  # [head, list, next index]
        while qi < len(queue) or active:
            while len(active) < slots and qi < len(queue):
                h, u = queue[qi]
                qi += 1
                key = (h, u)
                if key not in lists:
                    lists[key] = np.flatnonzero(m[h, u])
                if lists[key].size:
                    active.append([h, lists[key], 0])
            nxt = []
            for a in active:
                tile = (a[0], int(a[1][a[2]]))
                accesses += 1
                if tile in cache:
                    hits += 1
                    cache.move_to_end(tile)
                else:
                    cache[tile] = True
                    if len(cache) > lru_tiles:
                        cache.popitem(last=False)
                a[2] += 1
                if a[2] < a[1].size:
                    nxt.append(a)
            active = nxt
    return hits / accesses if accesses else 0.0
