"""The host-side locality proxies against brute force on small cases."""

import numpy as np

from cache_aware_query_amd import locality


def test_wave_objective_is_the_pairwise_distance_sum():
    rng = np.random.default_rng(1)
    m = (rng.random((2, 13, 20)) < 0.3).astype(np.uint8)
    perm = np.stack([rng.permutation(13) for _ in range(2)])
    want = 0
    for h in range(2):
        for _, lo, hi in locality._waves(13, 2, 3):
            rows = m[h, perm[h, lo:hi]].astype(np.int64)
            for i in range(len(rows)):
                for j in range(len(rows)):
                    want += int(((rows[i] - rows[j]) ** 2).sum())
    assert locality.wave_objective(m, perm, 2, 3) == want


def test_waves_follow_the_slices():
    # 10 rows, 3 slices of ceil(10/3) = 4 positions, waves of 3: [0,3) [3,4) [4,7) [7,8) [8,10)
    assert [(lo, hi) for _, lo, hi in locality._waves(10, 3, 3)] == [(0, 3), (3, 4), (4, 7),
                                                                     (7, 8), (8, 10)]


def test_distinct_blocks_per_wave():
    m = np.zeros((1, 4, 6), dtype=np.uint8)
    m[0, 0, [0, 1]] = 1
    m[0, 1, [1, 2]] = 1
    m[0, 2, [5]] = 1
    m[0, 3, [5]] = 1
    perm = np.array([[0, 1, 2, 3]])
    assert locality.distinct_kv_per_wave(m, perm, 1, 2) == (3 + 1) / 2
    perm = np.array([[0, 2, 1, 3]])
    assert locality.distinct_kv_per_wave(m, perm, 1, 2) == (3 + 3) / 2


def test_lru_model_hand_worked():
    # one XCD, two slots, LRU of 2 tiles.  Rows 0 {0, 1} and 1 {0, 1} run together:
    # step 0 both take tile 0 (miss, hit), step 1 tile 1 (miss, hit); row 2 {2} then
    # misses: 2 hits of 5 accesses.
    m = np.zeros((1, 3, 4), dtype=np.uint8)
    m[0, 0, [0, 1]] = 1
    m[0, 1, [0, 1]] = 1
    m[0, 2, [2]] = 1
    assert locality.lru_l2_model(m, np.array([[0, 1, 2]]), 1, slots=2, lru_tiles=2) == 2 / 5
    # one slot: each row alone; row 1 finds tiles 0 and 1 still cached
    assert locality.lru_l2_model(m, np.array([[0, 1, 2]]), 1, slots=1, lru_tiles=2) == 2 / 5
    # one slot and a one-tile cache: row 1 reads tile 0 (evicted by tile 1: miss),
    # then tile 1 (evicted by tile 0 just before: miss)
    assert locality.lru_l2_model(m, np.array([[0, 1, 2]]), 1, slots=1, lru_tiles=1) == 0.0
