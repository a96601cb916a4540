"""Pins of the MinHash comparator order (oracle/comparators.py) against the
definition of min-wise hashing: exact values of single-element rows, the subset
property, identical and empty rows, and the Jaccard estimate it is used for."""

import numpy as np

import oracle

P = (1 << 31) - 1


def test_single_element_rows_have_the_hash_value():
    m = np.zeros((3, 8), dtype=np.uint8)
    m[0, 7] = 1
    m[1, 5] = 1
    sig = oracle.minhash_signatures(m, [48271, (1 << 30) + 3], [11, 1])
    assert sig[0, 0] == 337908                     # 48271 * 7 + 11
    assert sig[1, 1] == 1073741842                 # ((2^30 + 3) * 5 + 1) mod (2^31 - 1)
    assert sig[2, 0] == P and sig[2, 1] == P       # empty row
    assert oracle.MINHASH_P == P


def test_signature_of_a_superset_is_not_larger():
    rng = np.random.default_rng(1)
    for _ in range(20):
        a = rng.random(64) < 0.2
        b = a | (rng.random(64) < 0.2)
        m = np.stack([a, b]).astype(np.uint8)
        ha = rng.integers(1, P, size=4)
        hb = rng.integers(0, P, size=4)
        sig = oracle.minhash_signatures(m, ha, hb)
        if a.any():
            assert np.all(sig[1] <= sig[0])


def test_identical_rows_are_neighbours_and_empty_rows_last():
    rng = np.random.default_rng(2)
    m = (rng.random((12, 40)) < 0.25).astype(np.uint8)
    m[9] = m[2]
    m[5] = 0
    perm = oracle.minhash_order_head(m, [1234567, 7654321], [3, 5], wave=4, n_slices=1,
                                     stage2=False)
    assert sorted(perm.tolist()) == list(range(12))
    pos = {int(r): i for i, r in enumerate(perm)}
    sig = oracle.minhash_signatures(m, [1234567, 7654321], [3, 5])
    lo, hi = sorted((pos[2], pos[9]))
    # nothing but rows with the very same signature can sit between two equal rows
    assert all(np.array_equal(sig[perm[i]], sig[2]) for i in range(lo, hi + 1))
    assert perm[-1] == 5


def test_equal_leading_hash_tracks_jaccard():
    """Agreement of one hash value estimates the Jaccard similarity.  Linear hashing
    mod P is only approximately min-wise independent on small integer sets, so the
    pin allows 0.1 of bias and checks the ordering of two pairs instead of equality."""
    rng = np.random.default_rng(3)
    def pair(lo_b, hi_b):
        a = np.zeros(200, dtype=bool)
        b = np.zeros(200, dtype=bool)
        a[:60] = True
        b[lo_b:hi_b] = True
        return np.stack([a, b]).astype(np.uint8)
    n = 3000
    ha = rng.integers(1, P, size=n)
    hb = rng.integers(0, P, size=n)
    fr = []
    for m, jac in ((pair(30, 100), 0.3), (pair(10, 70), 50 / 70)):
        sig = oracle.minhash_signatures(m, ha, hb)
        f = float(np.mean(sig[0] == sig[1]))
        assert abs(f - jac) < 0.1, (f, jac)
        fr.append(f)
    assert fr[1] > fr[0] + 0.25


def test_stage2_inside_buckets():
    rng = np.random.default_rng(4)
    mask = (rng.random((2, 30, 30)) < 0.3).astype(np.uint8)
    perm, inv = oracle.minhash_order(mask, [99991, 31337], [7, 8], wave=4, n_slices=2)
    for h in range(2):
        assert sorted(perm[h].tolist()) == list(range(30))
        assert np.array_equal(inv[h][perm[h]], np.arange(30))
        nnz = mask[h].sum(axis=1)
        base = oracle.minhash_order_head(mask[h], [99991, 31337], [7, 8], 4, 2, stage2=False)
        for lo, hi in oracle.wave_buckets(30, 2, 4):
            assert sorted(perm[h][lo:hi].tolist()) == sorted(base[lo:hi].tolist())
            assert list(-nnz[perm[h][lo:hi]]) == sorted(-nnz[perm[h][lo:hi]])


def test_signature_priority_hand_worked():
    """Hand-worked order with h1(v) = v and h2(v) = (P - 1) v + 5 mod P = 5 - v (for
    v <= 5), so sig1 = smallest id and sig2 = 5 - largest id <= 5:

        row 0 {3, 4}: (3, 1)    row 1 {1, 7}: (1, 4)
        row 2 {3, 5}: (3, 0)    row 3 {2}:    (2, 3)

    Sorted by sig1, then sig2, then row: 1, 3, 2, 0.  With sig2 primary the order
    would be 2, 0, 3, 1; with the row index before sig2 it would be 1, 3, 0, 2."""
    m = np.zeros((4, 8), dtype=np.uint8)
    for r, ids in enumerate(([3, 4], [1, 7], [3, 5], [2])):
        m[r, ids] = 1
    a, b = [1, P - 1], [0, 5]
    sig = oracle.minhash_signatures(m, a, b)
    assert sig.tolist() == [[3, 1], [1, 4], [3, 0], [2, 3]]
    order = oracle.minhash_order_head(m, a, b, wave=4, n_slices=1, stage2=False)
    assert order.tolist() == [1, 3, 2, 0]


def test_lsh_groups_hand_worked():
    """Two bands of two hashes.  Band 0: h(v) = v and h(v) = (P - 1) v + 9 (= 9 - v for
    v <= 9), i.e. (smallest id, 9 - largest id); band 1 uses the same two hashes in the
    other order, so it groups the same rows.

        row 0 {2, 5}: band 0 (2, 4)      row 1 {2, 5}: (2, 4)   (identical to row 0)
        row 2 {1, 3}: (1, 6)             row 3 {6}:    (6, 3)
        row 4 {1, 3, 8}: (1, 1)          row 5 {1, 3}: (1, 6)   (identical to row 2)

    Buckets shared: {0, 1} and {2, 5}; rows 3 and 4 alone.  Groups in order of their
    first row: [0, 1], [2, 5], [3], [4]."""
    m = np.zeros((6, 10), dtype=np.uint8)
    for r, ids in enumerate(([2, 5], [2, 5], [1, 3], [6], [1, 3, 8], [1, 3])):
        m[r, ids] = 1
    a = [1, P - 1, P - 1, 1]
    b = [0, 9, 9, 0]
    sig = oracle.minhash_signatures(m, a, b)
    assert sig[:, :2].tolist() == [[2, 4], [2, 4], [1, 6], [6, 3], [1, 1], [1, 6]]
    label = oracle.lsh_components(m, a, b, n_bands=2)
    assert label.tolist() == [0, 0, 2, 3, 4, 2]
    order = oracle.lsh_order_head(m, a, b, 2, wave=8, n_slices=1, stage2=False)
    assert order.tolist() == [0, 1, 2, 5, 3, 4]


def test_lsh_joins_directly_similar_rows_only():
    """Row 0 shares band 0 with row 1, row 1 shares band 1 with row 2, rows 0 and 2
    share nothing: row 1 joins row 0, row 2 joins row 1 (its lowest direct neighbour),
    not row 0 (no transitive closure)."""
    # band 0: (min id, min id); band 1: (9 - max id, 9 - max id) with h(v) = 9 - v
    a = [1, 1, P - 1, P - 1]
    b = [0, 0, 9, 9]
    m = np.zeros((4, 10), dtype=np.uint8)
    m[0, [0, 4]] = 1      # band 0 key (0, 0), band 1 key (5, 5)
    m[1, [0, 7]] = 1      # band 0 (0, 0) with row 0;  band 1 (2, 2)
    m[2, [3, 7]] = 1      # band 0 (3, 3);  band 1 (2, 2) with row 1
    m[3, [1, 2]] = 1      # band 0 (1, 1), band 1 (7, 7): alone
    label = oracle.lsh_components(m, a, b, n_bands=2)
    assert label.tolist() == [0, 0, 1, 3]
    # with band 0 alone row 2 joins nobody
    assert oracle.lsh_components(m, a, b, n_bands=1).tolist() == [0, 0, 2, 3]
    # order by (label, row): 0, 1 | 2 | 3 ... and a far row joins its group: move row 1's
    # lists to the end (row 3) and it still lands next to row 0
    m2 = m[[0, 3, 2, 1]]
    order = oracle.lsh_order_head(m2, a, b, 2, wave=8, n_slices=1, stage2=False)
    assert order.tolist() == [0, 3, 1, 2]


def test_lsh_identical_rows_share_a_group_and_empty_rows_group_together():
    rng = np.random.default_rng(5)
    m = (rng.random((30, 50)) < 0.2).astype(np.uint8)
    m[17] = m[4]
    m[9] = 0
    m[22] = 0
    ha = rng.integers(1, P, size=8)
    hb = rng.integers(0, P, size=8)
    label = oracle.lsh_components(m, ha, hb, n_bands=4)
    assert label[17] == label[4] and label[9] == label[22]
    assert all(label[u] <= u for u in range(30))
    perm, inv = oracle.lsh_order(m[None], ha, hb, 4, wave=4, n_slices=2)
    assert sorted(perm[0].tolist()) == list(range(30))
