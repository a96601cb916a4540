"""Pins of the reorder oracle (WaveAlign §IV, Algorithms 1 and 2).

* Eq. (2)/(3): centering keeps every pairwise row distance and zeroes the
  column sums; the distance splits over the singular triplets.
* Algorithm 1 against numpy.linalg.svd (a library routine) with many iterations.
* Closed forms: a circulant band mask has the frequency-1 Fourier pair as its
  top-2 centered subspace, so the polar order walks the rows cyclically; rows
  that are identical within clusters stay contiguous.
* Worked examples: Fig. 6 (polar order) and Fig. 7 (Stage-2 wave order), read
  from tests/golden.
* Stage-2 invariants and the skip rule's special cases.
"""

import numpy as np
import pytest

import oracle
from oracle.reorder import SKIP_ALWAYS, SKIP_NEVER


def _structured_mask(rng, mb=48, nb=40):
    """Rows near one of a few random 'centres' with noise: a top-heavy spectrum."""
    centres = (rng.random((4, nb)) < 0.3)
    rows = []
    for i in range(mb):
        r = centres[i % 4].copy()
        flip = rng.random(nb) < 0.05
        rows.append(r ^ flip)
    return np.array(rows, dtype=np.uint8)


def test_centering_preserves_distances_and_zeroes_column_sums():
    rng = np.random.default_rng(1)
    m = (rng.random((20, 15)) < 0.4).astype(np.uint8)
    mt = oracle.centered_mask(m)
    np.testing.assert_allclose(mt.sum(axis=0), 0.0, atol=1e-12)
    mf = m.astype(float)
    d0 = ((mf[:, None] - mf[None]) ** 2).sum(-1)
    d1 = ((mt[:, None] - mt[None]) ** 2).sum(-1)
    np.testing.assert_allclose(d1, d0, atol=1e-12)
    # eq. (3): the squared distance is the sigma^2-weighted distance of the left vectors
    u, s, _ = np.linalg.svd(mt)
    r = len(s)
    d3 = (((u[:, None, :r] - u[None, :, :r]) ** 2) * s[None, None] ** 2).sum(-1)
    np.testing.assert_allclose(d3, d0, atol=1e-10)


def _principal_sin(a, b):
    # sine of the largest principal angle as the norm of b's part outside span(a):
    # ||(I - Qa Qa^T) Qb||_2 resolves angles down to rounding, unlike sqrt(1 - cos^2)
    qa, _ = np.linalg.qr(a)
    qb, _ = np.linalg.qr(b)
    return float(np.linalg.norm(qb - qa @ (qa.T @ qb), 2))


def test_mfcsi_matches_library_svd():
    rng = np.random.default_rng(2)
    m = _structured_mask(rng)
    u, s, _ = np.linalg.svd(oracle.centered_mask(m))
    assert s[1] / s[2] >= 1.05
    x0 = rng.uniform(-1, 1, size=(m.shape[0], 2))
    got = oracle.mfcsi(m, x0, iters=200)
    assert _principal_sin(got, u[:, :2]) < 1e-8
    # Ritz ordering: the first column is the leading singular vector (up to sign)
    assert abs(abs(got[:, 0] @ u[:, 0]) - 1.0) < 1e-8
    np.testing.assert_allclose(got.T @ got, np.eye(2), atol=1e-12)


def test_mfcsi_circulant_band_gives_cyclic_order():
    n, half = 64, 3
    m = np.zeros((n, n), dtype=np.uint8)
    for i in range(n):
        for off in range(-half, half + 1):
            m[i, (i + off) % n] = 1
    rng = np.random.default_rng(3)
    got = oracle.mfcsi(m, rng.uniform(-1, 1, size=(n, 2)), iters=300)
    theta = 2 * np.pi * np.arange(n) / n
    fourier = np.stack([np.cos(theta), np.sin(theta)], axis=1)
    assert _principal_sin(got, fourier) < 1e-6
    order = oracle.stage1_order(oracle.polar_angles(got))
    steps = np.diff(np.concatenate([order, order[:1]])) % n
    assert np.all(steps == 1) or np.all(steps == n - 1)


def test_identical_row_clusters_stay_contiguous():
    rng = np.random.default_rng(4)
    nb = 30
    centres = (rng.random((3, nb)) < 0.4).astype(np.uint8)
    labels = rng.permutation(np.repeat(np.arange(3), [7, 11, 9]))
    m = centres[labels]
    got = oracle.mfcsi(m, rng.uniform(-1, 1, size=(len(labels), 2)), iters=20)
    order = oracle.stage1_order(oracle.polar_angles(got))
    seq = labels[order]
    changes = int(np.sum(seq[1:] != seq[:-1]))
    assert changes == 2


def test_fig6_polar_order(golden):
    g = golden("fig6_polar_order.txt")
    u = np.stack([np.array(g["u1"], float), np.array(g["u2"], float)], axis=1)
    order = oracle.stage1_order(oracle.polar_angles(u))
    assert order.tolist() == [int(x) for x in g["order"]]


def test_fig7_stage2_wave_order(golden):
    g = golden("fig7_stage2.txt")
    nnz = np.array(g["nnz"], dtype=np.int64)
    w = int(g["wave"][0])
    perm = oracle.stage2_order(np.arange(len(nnz)), nnz, oracle.wave_buckets(len(nnz), 1, w))
    assert perm[:w].tolist() == [int(x) for x in g["wave0"]]
    head = [int(x) for x in g["wave1_head"]]
    assert perm[w:w + len(head)].tolist() == head
    assert sorted(perm[w:2 * w].tolist()) == list(range(w, 2 * w))


def test_stage2_invariants_and_slices():
    rng = np.random.default_rng(5)
    mb = 591
    nnz = rng.integers(1, 200, size=mb)
    order = rng.permutation(mb)
    for n_slices, wave in ((1, 64), (8, 64), (8, 32), (3, 7)):
        buckets = oracle.wave_buckets(mb, n_slices, wave)
        assert buckets[0][0] == 0 and buckets[-1][1] == mb
        assert all(b[1] == c[0] for b, c in zip(buckets, buckets[1:]))
        assert all(0 < hi - lo <= wave for lo, hi in buckets)
        perm = oracle.stage2_order(order, nnz, buckets)
        assert sorted(perm.tolist()) == list(range(mb))
        for lo, hi in buckets:
            assert sorted(perm[lo:hi].tolist()) == sorted(order[lo:hi].tolist())
            assert np.all(np.diff(nnz[perm[lo:hi]]) <= 0)
    # 8 slices of ceil(591/8) = 74 positions, each cut at 64
    b8 = oracle.wave_buckets(mb, 8, 64)
    assert b8[:3] == [(0, 64), (64, 74), (74, 138)]
    assert b8[-1] == (582, 591)


def test_rank_one_centered_mask_splits_by_sign():
    # Two distinct row types: the centered mask has rank one, the second basis
    # vector is zero and the angles take only the values 0 and pi.
    rng = np.random.default_rng(6)
    a = rng.random(50) < 0.4
    b = rng.random(50) < 0.4
    labels = (rng.random(200) < 0.3).astype(int)
    m = np.where(labels[:, None] == 1, a, b).astype(np.uint8)
    got = oracle.mfcsi(m, rng.uniform(-1, 1, (200, 2)), iters=10)
    assert np.all(got[:, 1] == 0.0)
    ang = oracle.polar_angles(got)
    assert set(np.round(ang, 12).tolist()) <= {0.0, round(np.pi, 12)}
    seq = labels[oracle.stage1_order(ang)]
    assert int(np.sum(seq[1:] != seq[:-1])) == 1


def test_explicit_iteration_equals_the_matrix_free_form():
    # The oracle forms M~ = M - 1 c^T / MB explicitly.  The same products can be taken
    # with the 0/1 mask and rank-1 corrections (c = M^T 1):
    #   M~^T X = M^T X - c (1^T X) / MB,   M~ Y = M Y - 1 (c^T Y) / MB,
    # which never forms M~; with a library QR both give the same basis.
    rng = np.random.default_rng(10)
    m = _structured_mask(rng, 60, 50).astype(np.float64)
    x0 = rng.uniform(-1, 1, (60, 2))
    c = m.sum(axis=0)
    ones = np.ones(60)
    x, _ = np.linalg.qr(x0)
    for _ in range(3):
        y = m.T @ x - np.outer(c, ones @ x) / 60
        z = m @ y - np.outer(ones, c @ y) / 60
        x, r = np.linalg.qr(z)
        x = x * np.sign(np.diag(r))[None, :]
    want = oracle.canonical_signs(x)
    got = oracle.mfcsi(m, x0, iters=3, ritz=False)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_ritz_step_diagonalises_and_orders():
    rng = np.random.default_rng(11)
    m = _structured_mask(rng, 60, 50)
    got = oracle.mfcsi(m, rng.uniform(-1, 1, (60, 2)), iters=10)
    mt = oracle.centered_mask(m)
    bmat = got.T @ mt @ mt.T @ got
    assert abs(bmat[0, 1]) < 1e-9 * abs(bmat[0, 0])
    assert bmat[0, 0] >= bmat[1, 1]
    # sign convention: positive sum of cubes per column
    assert np.all(np.sum(got ** 3, axis=0) > 0)


def test_identical_rows_and_skip_rule():
    m = np.ones((16, 16), dtype=np.uint8)
    assert oracle.mfcsi(m, np.ones((16, 2)), 10) is None
    st = oracle.skip_statistics(m, 128, 128)
    assert st[0] == 256 and st[1] == 1.0 and st[4] == 1.0
    assert st[2] == 16 * 128 * 128 * 4 and st[3] == 4.0 * 128 * 128 * 128 * 256
    p = oracle.ReorderParams(ws_min_bytes=0.0, flops_min=0.0, jaccard_max=0.9)
    assert oracle.skip_decision(st, p)                  # already local (dense)
    perm, skipped, _, _ = oracle.reorder_head(m, np.ones((16, 2)), 128, 128, p)
    assert skipped and perm.tolist() == list(range(16))
    rng = np.random.default_rng(7)
    r = (rng.random((16, 16)) < 0.3).astype(np.uint8)
    st = oracle.skip_statistics(r, 128, 128)
    assert not oracle.skip_decision(st, p)
    assert oracle.skip_decision(st, oracle.ReorderParams(ws_min_bytes=st[2]))      # fits the cache
    assert oracle.skip_decision(st, oracle.ReorderParams(flops_min=st[3] + 1))     # too little work
    assert not oracle.skip_decision(st, oracle.ReorderParams(flops_min=st[3]))
    assert oracle.skip_decision(st, oracle.ReorderParams(skip_mode=SKIP_ALWAYS))
    assert not oracle.skip_decision(oracle.skip_statistics(m, 128, 128),
                                    oracle.ReorderParams(skip_mode=SKIP_NEVER, jaccard_max=0.0))


def test_work_case_is_decided_per_call():
    """The work case looks at the heaviest head of the call: a light head is
    reordered when a heavier head of the same call pays for the launch, and every
    head keeps its order when none does."""
    rng = np.random.default_rng(11)
    heavy = (rng.random((24, 24)) < 0.5).astype(np.uint8)
    light = np.zeros((24, 24), dtype=np.uint8)
    light[np.arange(24), rng.integers(0, 24, 24)] = 1     # one block per row
    light[np.arange(0, 24, 2), rng.integers(0, 24, 12)] = 1
    mask = np.stack([heavy, light])
    x0 = rng.standard_normal((2, 24, 2))
    f_heavy = 4.0 * 64 * 64 * 64 * int(heavy.sum())
    f_light = 4.0 * 64 * 64 * 64 * int(light.sum())
    assert f_light < f_heavy
    p = oracle.ReorderParams(wave=8, n_slices=1, flops_min=(f_light + f_heavy) / 2, jaccard_max=1.0)
    # alone, the light head is below the threshold ...
    assert oracle.skip_decision(oracle.skip_statistics(light, 64, 64), p)
    assert oracle.reorder_head(light, x0[1], 64, 64, p)[1]
    # ... beside the heavy head, in one call, it is reordered
    _, _, skipped, _, st = oracle.reorder_rows(mask, x0, 64, 64, p)
    assert st[1, 3] == f_light and st[0, 3] == f_heavy
    assert skipped.tolist() == [False, False]
    # a threshold above the heaviest head skips both
    p_hi = oracle.ReorderParams(wave=8, n_slices=1, flops_min=f_heavy + 1, jaccard_max=1.0)
    assert oracle.reorder_rows(mask, x0, 64, 64, p_hi)[2].tolist() == [True, True]


def test_jaccard_is_pooled_over_adjacent_rows():
    m = np.array([[1, 1, 0, 0], [0, 1, 1, 0], [0, 0, 0, 0], [1, 1, 1, 1]], dtype=np.uint8)
    st = oracle.skip_statistics(m, 64, 64)
    # pairs: (0,1) inter 1 union 3; (1,2) inter 0 union 2; (2,3) inter 0 union 4
    assert st[4] == pytest.approx(1.0 / 9.0, abs=0)


def test_start_block_does_not_change_converged_order():
    rng = np.random.default_rng(8)
    m = _structured_mask(rng, 40, 36)
    a = oracle.polar_angles(oracle.mfcsi(m, rng.uniform(-1, 1, (40, 2)), 300))
    b = oracle.polar_angles(oracle.mfcsi(m, -rng.uniform(-1, 1, (40, 2)), 300))
    np.testing.assert_allclose(a, b, atol=1e-7)


def test_reorder_rows_outputs_are_consistent():
    rng = np.random.default_rng(9)
    H, mb = 3, 50
    mask = np.stack([_structured_mask(rng, mb, 45) for _ in range(H)])
    x0 = rng.uniform(-1, 1, (H, mb, 2))
    p = oracle.ReorderParams(wave=8, n_slices=2, skip_mode=SKIP_NEVER)
    perm, inv, skipped, angles, stats = oracle.reorder_rows(mask, x0, 64, 64, p)
    assert not skipped.any()
    for h in range(H):
        assert sorted(perm[h].tolist()) == list(range(mb))
        np.testing.assert_array_equal(inv[h][perm[h]], np.arange(mb))
        assert np.all(np.isfinite(angles[h]))
        # with Stage 2 off the permutation is the plain angle order
    p1 = oracle.ReorderParams(wave=8, n_slices=2, skip_mode=SKIP_NEVER, stage2=False)
    perm1, _, _, angles1, _ = oracle.reorder_rows(mask, x0, 64, 64, p1)
    for h in range(H):
        np.testing.assert_array_equal(perm1[h], np.argsort(angles1[h], kind="stable"))
