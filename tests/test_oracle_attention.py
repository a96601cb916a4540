"""Pins of the fp64 attention oracle against definitions it does not share code with.

* All-ones mask: torch's scaled_dot_product_attention in fp64 (a library routine).
* Per-element brute force with Python loops on tiny inputs.
* Row LSE against scipy.special.logsumexp of the explicit score matrix.
* Invariants from the pages: a fully masked row gives O = 0 and LSE = -inf
  (GSRS, fully masked rows); the output does not change when query blocks are
  permuted (WaveAlign §IV-A: rows are independent, so reordering preserves the
  semantics); padded keys never enter a softmax.
"""

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_ones_mask_equals_library_attention():
    H, L, d, b = 2, 256, 32, 64
    q, k, v = (_rand((H, L, d), s) for s in (1, 2, 3))
    mask = np.ones((H, L // b, L // b), dtype=np.uint8)
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, 1.0 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    z = np.einsum("hid,hjd->hij", q, k) / math.sqrt(d)
    np.testing.assert_allclose(lse, logsumexp(z, axis=2), rtol=0, atol=1e-12)


def _brute(q, k, v, mask, L, b, s):
    H, lp, d = q.shape
    o = np.full((H, lp, d), np.nan)
    lse = np.full((H, lp), np.nan)
    for h in range(H):
        for i in range(L):
            zs, vs = [], []
            for j in range(L):
                if mask[h][i // b][j // b]:
                    acc = 0.0
                    for c in range(d):
                        acc += q[h][i][c] * k[h][j][c]
                    zs.append(s * acc)
                    vs.append(j)
            if not zs:
                o[h, i] = 0.0
                lse[h, i] = -math.inf
                continue
            mx = max(zs)
            den = sum(math.exp(z - mx) for z in zs)
            lse[h, i] = mx + math.log(den)
            for c in range(d):
                o[h, i, c] = sum(math.exp(z - mx) / den * v[h][j][c] for z, j in zip(zs, vs))
    return o, lse


def test_brute_force_tiny_ragged_with_empty_row():
    H, L, d, b = 2, 40, 4, 16          # 3 blocks, the last has 8 valid tokens
    lp = 48
    q, k, v = (np.zeros((H, lp, d)) for _ in range(3))
    for t, s in zip((q, k, v), (4, 5, 6)):
        t[:, :L] = _rand((H, L, d), s)
    mask = np.array([[[1, 0, 1], [0, 0, 0], [1, 1, 0]],
                     [[0, 1, 1], [1, 0, 0], [1, 1, 1]]], dtype=np.uint8)
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, 0.7)
    ob, lb = _brute(q, k, v, mask, L, b, 0.7)
    np.testing.assert_allclose(o[:, :L], ob[:, :L], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse[:, :L]), np.isneginf(lb[:, :L]))
    fin = np.isfinite(lb[:, :L])
    np.testing.assert_allclose(lse[:, :L][fin], lb[:, :L][fin], rtol=0, atol=1e-12)
    assert np.all(np.isnan(o[:, L:]))


def test_fully_masked_row_is_zero_and_neg_inf():
    H, L, d, b = 1, 128, 8, 32
    q, k, v = (_rand((H, L, d), s) for s in (7, 8, 9))
    mask = np.ones((H, 4, 4), dtype=np.uint8)
    mask[0, 2] = 0
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, 0.3)
    assert np.all(o[0, 64:96] == 0.0)
    assert np.all(np.isneginf(lse[0, 64:96]))
    assert np.all(np.isfinite(lse[0, :64]))


def test_padded_keys_never_attend():
    H, L, d, b = 1, 300, 16, 64         # L_pad = 320
    lp = 320
    q, k, v = (np.zeros((H, lp, d)) for _ in range(3))
    for t, s in zip((q, k, v), (10, 11, 12)):
        t[:, :L] = _rand((H, L, d), s)
    mask = np.ones((H, 5, 5), dtype=np.uint8)
    s = 1.0 / math.sqrt(d)
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, s)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, :L]), torch.from_numpy(k[:, :L]), torch.from_numpy(v[:, :L])).numpy()
    np.testing.assert_allclose(o[:, :L], ref, rtol=0, atol=1e-12)
    k2, v2 = k.copy(), v.copy()
    k2[:, L:] = 5.0
    v2[:, L:] = -3.0
    o2, _ = oracle.masked_attention(q, k2, v2, mask, L, b, s)
    np.testing.assert_array_equal(o[:, :L], o2[:, :L])


def test_single_block_row_equals_attention_on_that_block():
    H, L, d, b = 1, 256, 16, 64
    q, k, v = (_rand((H, L, d), s) for s in (13, 14, 15))
    mask = np.zeros((H, 4, 4), dtype=np.uint8)
    mask[0, 1, 3] = 1
    o, _ = oracle.masked_attention(q, k, v, mask, L, b, 1.0 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, 64:128]), torch.from_numpy(k[:, 192:256]),
        torch.from_numpy(v[:, 192:256])).numpy()
    np.testing.assert_allclose(o[:, 64:128], ref, rtol=0, atol=1e-12)


def test_query_block_permutation_invariance():
    H, L, d, b = 2, 320, 8, 32
    q, k, v = (_rand((H, L, d), s) for s in (16, 17, 18))
    rng = np.random.default_rng(19)
    mask = (rng.random((H, 10, 10)) < 0.4).astype(np.uint8)
    s = 0.25
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, s)
    perm = np.stack([rng.permutation(10) for _ in range(H)])
    qp = oracle.gather_blocks(q, perm, b)
    mp = np.stack([mask[h][perm[h]] for h in range(H)])
    op, lp_ = oracle.masked_attention(qp, k, v, mp, L, b, s)
    np.testing.assert_array_equal(oracle.scatter_blocks(op, perm, b), o)
    np.testing.assert_array_equal(oracle.scatter_blocks(lp_[..., None], perm, b)[..., 0], lse)


def test_rows_subset_matches_full():
    H, L, d, b = 1, 200, 8, 64
    q, k, v = (_rand((H, 256, d), s) for s in (20, 21, 22))
    rng = np.random.default_rng(23)
    mask = (rng.random((H, 4, 4)) < 0.6).astype(np.uint8)
    o, lse = oracle.masked_attention(q, k, v, mask, L, b, 0.4)
    rows = np.array([0, 63, 64, 130, 199])
    o2, l2 = oracle.masked_attention_rows(q[0], k[0], v[0], mask[0], rows, L, b, 0.4)
    np.testing.assert_allclose(o2, o[0, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lse[0, rows], rtol=0, atol=1e-14)


def test_entropy_closed_forms_and_scipy():
    from scipy.stats import entropy as sp_entropy

    H, L, d, b = 1, 150, 8, 32
    nb = -(-L // b)
    lp = nb * b
    mask = np.ones((H, nb, nb), dtype=np.uint8)
    mask[0, 1] = 0                       # an empty row block
    mask[0, 2] = 0
    mask[0, 2, 4] = 1                    # the last, ragged block alone: 150 - 128 = 22 keys
    # Zero queries: uniform attention over the allowed keys, entropy ln(#keys).
    q0 = np.zeros((H, lp, d))
    k = np.zeros((H, lp, d))
    k[:, :L] = _rand((H, L, d), 7)
    ent = oracle.attention_entropy(q0, k, mask, L, b, 1.0)
    assert np.allclose(ent[0, :b], math.log(L), atol=1e-12)
    assert np.all(ent[0, b:2 * b] == 0.0)
    assert np.allclose(ent[0, 2 * b:3 * b], math.log(L - 4 * b), atol=1e-12)
    assert np.all(np.isnan(ent[0, L:]))
    # Random queries: scipy's entropy of the explicit probabilities.
    q = np.zeros((H, lp, d))
    q[:, :L] = _rand((H, L, d), 8)
    s = 1.0 / math.sqrt(d)
    ent = oracle.attention_entropy(q, k, mask, L, b, s)
    for i in (0, 5, 31, 70, 100, 149):
        u = i // b
        keys = [j for j in range(L) if mask[0, u, j // b]]
        if not keys:
            continue
        z = s * np.array([q[0, i] @ k[0, j] for j in keys])
        p = np.exp(z - logsumexp(z))
        assert abs(ent[0, i] - sp_entropy(p)) < 1e-12
    # A dominant key drives the entropy to zero.
    qd = q.copy()
    qd[0, 0] = 200.0 * k[0, 3]
    assert oracle.attention_entropy(qd, k, mask, L, b, s)[0, 0] < 1e-6


def test_distance_closed_forms_and_brute_force():
    H, L, d, b = 1, 150, 8, 32
    nb = -(-L // b)
    lp = nb * b
    mask = np.ones((H, nb, nb), dtype=np.uint8)
    mask[0, 1] = 0                       # an empty row block
    mask[0, 2] = 0
    mask[0, 2, 4] = 1                    # keys 128..149 only: all to the right of rows 64..95
    q0 = np.zeros((H, lp, d))
    k = np.zeros((H, lp, d))
    k[:, :L] = _rand((H, L, d), 9)
    dist = oracle.attention_distance(q0, k, mask, L, b, 1.0)
    # Uniform weights over all L keys: the mean of |i - j| over j, summed as two series.
    for i in range(b):
        assert abs(dist[0, i] - (i * (i + 1) / 2 + (L - 1 - i) * (L - i) / 2) / L) < 1e-10
    assert np.all(dist[0, b:2 * b] == 0.0)
    for i in range(2 * b, 3 * b):
        assert abs(dist[0, i] - ((128 + 149) / 2 - i)) < 1e-10
    assert np.all(np.isnan(dist[0, L:]))
    # Random queries: explicit weights and distances, one key at a time.
    q = np.zeros((H, lp, d))
    q[:, :L] = _rand((H, L, d), 10)
    s = 1.0 / math.sqrt(d)
    dist = oracle.attention_distance(q, k, mask, L, b, s)
    for i in (0, 5, 31, 70, 100, 149):
        keys = [j for j in range(L) if mask[0, i // b, j // b]]
        if not keys:
            continue
        z = [s * sum(q[0, i, c] * k[0, j, c] for c in range(d)) for j in keys]
        zm = max(z)
        w = [math.exp(x - zm) for x in z]
        tot = sum(w)
        ref = sum(wj / tot * abs(i - j) for wj, j in zip(w, keys))
        assert abs(dist[0, i] - ref) < 1e-9
    # A dominant key: the distance tends to |i - j*|.
    qd = q.copy()
    qd[0, 7] = 200.0 * k[0, 120]
    assert abs(oracle.attention_distance(qd, k, mask, L, b, s)[0, 7] - 113.0) < 1e-6
