"""Pins of the block-index oracle: brute-force loops and a round trip to the mask."""

import numpy as np

import oracle


def test_block_index_brute_force_and_round_trip():
    rng = np.random.default_rng(0)
    H, MB, NB = 3, 7, 9
    mask = (rng.random((H, MB, NB)) < 0.35).astype(np.uint8)
    mask[1, 4] = 0                       # an empty row
    mask[2, :, 5] = 0                    # an empty column
    row_ptr, col_idx, row_nnz, csc_ptr, csc_idx = oracle.block_index(mask)
    # brute force
    pos = 0
    for h in range(H):
        for u in range(MB):
            assert row_ptr[h * MB + u] == pos
            cnt = 0
            for v in range(NB):
                if mask[h, u, v]:
                    assert col_idx[pos] == v
                    pos += 1
                    cnt += 1
            assert row_nnz[h * MB + u] == cnt
    assert row_ptr[-1] == pos == mask.sum()
    pos = 0
    for h in range(H):
        for v in range(NB):
            assert csc_ptr[h * NB + v] == pos
            for u in range(MB):
                if mask[h, u, v]:
                    assert csc_idx[pos] == u
                    pos += 1
    # round trip
    back = np.zeros_like(mask)
    for r in range(H * MB):
        h, u = divmod(r, MB)
        back[h, u, col_idx[row_ptr[r]:row_ptr[r + 1]]] = 1
    np.testing.assert_array_equal(back, mask)


def test_block_index_empty_mask():
    mask = np.zeros((2, 3, 4), dtype=np.uint8)
    row_ptr, col_idx, row_nnz, csc_ptr, csc_idx = oracle.block_index(mask)
    assert row_ptr.tolist() == [0] * 7
    assert col_idx.size == 0 and csc_idx.size == 0
    assert csc_ptr.tolist() == [0] * 9
