"""Pins of the GSRS oracle (fused block importance and Top-p).

* sum_v W_uv = 1 for every query block with a non-empty candidate set (GSRS,
  Appendix A.2).
* W from G and the row LSE equals W computed from explicit attention
  probabilities (the definition of block importance).
* G and the row LSE against scipy.special.logsumexp; log sum_v exp(G_iv) = L_i.
* Negative test: a stale row normaliser (AdaSpa's cached LSE) gives per-row
  sums exp(L_i - L_i_old) != 1.
* Top-p: brute force over prefixes, one-hot and uniform weights, p = 1 keeps
  everything, a second selection restricted to the first selection is a subset.
"""

import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def _case(seed, H=2, L=200, d=16, b=32, density=0.5, empty=(2,)):
    rng = np.random.default_rng(seed)
    nb = -(-L // b)
    lp = nb * b
    q, k = (np.zeros((H, lp, d)) for _ in range(2))
    q[:, :L] = rng.standard_normal((H, L, d)) * 1.5
    k[:, :L] = rng.standard_normal((H, L, d))
    mask = (rng.random((H, nb, nb)) < density).astype(np.uint8)
    for r in empty:
        mask[:, r] = 0
    return q, k, mask, L, b, 1.0 / math.sqrt(d)


def test_block_weights_sum_to_one_and_match_probabilities():
    q, k, mask, L, b, s = _case(1)
    row_ptr, col_idx, _, _, _ = oracle.block_index(mask)
    g, lse = oracle.block_lse(q, k, row_ptr, col_idx, L, b, s)
    w = oracle.block_importance(g, lse, row_ptr, L, b)
    wp = oracle.block_importance_from_probs(q, k, row_ptr, col_idx, L, b, s)
    np.testing.assert_allclose(w, wp, rtol=0, atol=1e-13)
    H, mb = mask.shape[0], mask.shape[1]
    for r in range(H * mb):
        lo, hi = row_ptr[r], row_ptr[r + 1]
        if hi > lo:
            assert abs(w[lo:hi].sum() - 1.0) < 1e-12
    # the empty query block has -inf LSE on its valid rows
    assert np.all(np.isneginf(lse[:, 2 * b:3 * b]))


def test_block_lse_against_logsumexp():
    q, k, mask, L, b, s = _case(2, H=1, L=150, empty=())
    row_ptr, col_idx, _, _, _ = oracle.block_index(mask)
    g, lse = oracle.block_lse(q, k, row_ptr, col_idx, L, b, s)
    mb = mask.shape[1]
    for u in range(mb):
        r0, r1 = u * b, min((u + 1) * b, L)
        lo, hi = row_ptr[u], row_ptr[u + 1]
        if hi == lo:
            continue
        for e in range(lo, hi):
            v = col_idx[e]
            keys = np.arange(v * b, min((v + 1) * b, L))
            z = s * q[0, r0:r1] @ k[0, keys].T
            np.testing.assert_allclose(g[e, :r1 - r0], logsumexp(z, axis=1), rtol=0, atol=1e-12)
        np.testing.assert_allclose(logsumexp(g[lo:hi, :r1 - r0], axis=0), lse[0, r0:r1],
                                   rtol=0, atol=1e-12)
    # the row LSE is the attention oracle's LSE
    _, lse2 = oracle.masked_attention(q, k, k, mask, L, b, s)
    np.testing.assert_allclose(lse[0, :L], lse2[0, :L], rtol=0, atol=1e-12)


def test_cached_lse_scores_do_not_sum_to_one():
    q, k, mask, L, b, s = _case(3, H=1, empty=())
    row_ptr, col_idx, _, _, _ = oracle.block_index(mask)
    g, lse = oracle.block_lse(q, k, row_ptr, col_idx, L, b, s)
    _, lse_old = oracle.block_lse(q * 0.8, k, row_ptr, col_idx, L, b, s)
    sc = oracle.cached_lse_scores(g, lse_old, row_ptr, L, b)
    mb = mask.shape[1]
    u = int(np.flatnonzero(np.diff(row_ptr) > 0)[0])
    r0 = u * b
    rowsum = np.nansum(sc[row_ptr[u]:row_ptr[u + 1]], axis=0)[:b]
    alpha = np.exp(lse[0, r0:r0 + b] - lse_old[0, r0:r0 + b])
    np.testing.assert_allclose(rowsum, alpha, rtol=1e-12)
    assert np.max(np.abs(rowsum - 1.0)) > 1e-3
    assert mb > 0


def _brute_topp(w, p):
    """Shortest prefix of the sorted order whose sum exceeds p (all if none)."""
    order = sorted(range(len(w)), key=lambda j: (-w[j], j))
    for n in range(1, len(order) + 1):
        total = 0.0
        for j in order[:n]:
            total += float(w[j])
        if total > p:
            return set(order[:n])
    return set(order)


def _one_row(w, p):
    w = np.asarray(w, dtype=np.float32)
    row_ptr = np.array([0, len(w)])
    col = np.arange(len(w))
    m = oracle.topp_select(w, row_ptr, col, 1, 1, len(w), p)
    return set(np.flatnonzero(m[0, 0]).tolist())


def test_topp_against_prefix_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(200):
        n = int(rng.integers(1, 12))
        w = rng.random(n).astype(np.float32)
        if trial % 3 == 0:
            w[rng.integers(0, n, size=n // 2)] = w[0]      # ties
        w = (w / w.sum()).astype(np.float32)
        p = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95]))
        assert _one_row(w, p) == _brute_topp(w, p)


def test_topp_special_cases():
    assert _one_row([0, 0, 1, 0], 0.9) == {2}
    assert _one_row([0.25, 0.25, 0.25, 0.25], 1.0) == {0, 1, 2, 3}
    # equal weights: ties go to the lower block id
    assert _one_row([0.25, 0.25, 0.25, 0.25], 0.3) == {0, 1}
    # exactly p after two blocks: "exceeds p" needs the third
    assert _one_row([0.25, 0.25, 0.25, 0.25], 0.5) == {0, 1, 2}
    # uniform float32 weights: the fp64 running sum of float32(1/100) stays below 0.9
    # after 90 blocks, so the 91st is the one that crosses
    assert len(_one_row([np.float32(0.01)] * 100, 0.9)) == 91


def test_topp_restricted_to_candidates_is_subset():
    q, k, mask, L, b, s = _case(5, H=2, L=256, density=0.7, empty=())
    row_ptr, col_idx, _, _, _ = oracle.block_index(mask)
    g, lse = oracle.block_lse(q, k, row_ptr, col_idx, L, b, s)
    w = oracle.block_importance(g, lse, row_ptr, L, b).astype(np.float32)
    H, mb, nb = mask.shape
    s1 = oracle.topp_select(w, row_ptr, col_idx, H, mb, nb, 0.9)
    assert np.all(s1 <= mask)
    rp1, ci1, _, _, _ = oracle.block_index(s1)
    g1, l1 = oracle.block_lse(q, k, rp1, ci1, L, b, s)
    w1 = oracle.block_importance(g1, l1, rp1, L, b).astype(np.float32)
    s2 = oracle.topp_select(w1, rp1, ci1, H, mb, nb, 0.8)
    assert np.all(s2 <= s1)
    assert s2.sum() < s1.sum()


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_topp_extremes(p):
    w = np.array([0.1, 0.6, 0.3], dtype=np.float32)
    got = _one_row(w, p)
    assert got == ({1} if p == 0.0 else {0, 1, 2})


def _dense_recall(q, k, mask, L, b, s):
    """Recall from the whole L x L attention matrix and the element mask it expands to."""
    H, lp, _ = q.shape
    nb = lp // b
    out = np.zeros((H, nb))
    for h in range(H):
        z = s * np.einsum("id,jd->ij", q[h, :L], k[h, :L])
        a = np.exp(z - logsumexp(z, axis=1, keepdims=True))
        m = np.kron(mask[h], np.ones((b, b)))[:L, :L]
        per_row = (a * m).sum(axis=1)
        for u in range(nb):
            out[h, u] = per_row[u * b:min((u + 1) * b, L)].mean()
    return out


def test_mask_recall_definition_and_identities():
    q, k, mask, L, b, s = _case(6, L=230, empty=(1,))
    H, nb = mask.shape[0], mask.shape[1]
    rec = oracle.mask_recall(q, k, mask, L, b, s)
    np.testing.assert_allclose(rec, _dense_recall(q, k, mask, L, b, s), rtol=0, atol=1e-13)
    ones = np.ones_like(mask)
    np.testing.assert_allclose(oracle.mask_recall(q, k, ones, L, b, s), 1.0, rtol=0, atol=1e-12)
    assert np.all(oracle.mask_recall(q, k, np.zeros_like(mask), L, b, s) == 0.0)
    # additive over disjoint masks
    other = (ones - mask).astype(np.uint8)
    tot = rec + oracle.mask_recall(q, k, other, L, b, s)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-12)
    # equals the sum of the full pass's block weights over the kept blocks (GSRS eq. (5))
    rp, ci, _, _, _ = oracle.block_index(ones)
    wfull = oracle.block_importance_from_probs(q, k, rp, ci, L, b, s)
    for h in range(H):
        for u in range(nb):
            lo = rp[h * nb + u]
            kept = sum(wfull[lo + v] for v in range(nb) if mask[h, u, v])
            assert abs(kept - rec[h, u]) < 1e-12


def _static_qk(seed=5, H=2, L=600, d=32, b=64):
    rng = np.random.default_rng(seed)
    mb = -(-L // b)
    q = np.zeros((H, mb * b, d))
    k = np.zeros((H, mb * b, d))
    q[:, :L] = rng.standard_normal((H, L, d)) * 2.0
    k[:, :L] = rng.standard_normal((H, L, d)) * 2.0
    return q, k, L, b, d ** -0.5


def test_schedule_steps_follow_warmup_search_and_reuse():
    """The control flow of the schedule: dense warmup, searches at T, reuse of the
    latest search's mask in between (GSRS §4-5)."""
    q, k, L, b, scale = _static_qk()
    kinds, masks, weights = oracle.gsrs_schedule(9, (2, 5, 7), (0.9, 0.5, 0.6),
                                                 lambda t: (q, k), L, b, scale)
    assert kinds == ["warmup", "warmup", "search", "reuse", "reuse", "search", "reuse",
                     "search", "reuse"]
    assert sorted(weights) == [2, 5, 7]
    assert np.all(masks[0] == 1) and np.all(masks[1] == 1)
    # reuse steps run the latest search's mask, not the candidate set
    assert np.array_equal(masks[3], masks[2]) and np.array_equal(masks[4], masks[2])
    assert np.array_equal(masks[6], masks[5]) and np.array_equal(masks[8], masks[7])
    assert not np.array_equal(masks[6], masks[2])


def test_reduced_search_stays_inside_the_candidate_set():
    """Later searches select among S1 only: with a small first threshold and a large
    later one, a search over all blocks would keep blocks outside S1."""
    q, k, L, b, scale = _static_qk(seed=6)
    kinds, masks, weights = oracle.gsrs_schedule(4, (1, 2), (0.3, 0.99),
                                                 lambda t: (q, k), L, b, scale)
    s1 = masks[1]
    assert np.all(masks[2] <= s1) and np.all(masks[3] <= s1)
    # W at the second search is normalised over S1: each row's weights sum to one
    rp, _, _, _, _ = oracle.block_index(s1)
    w = weights[2]
    for r in range(len(rp) - 1):
        if rp[r + 1] > rp[r]:
            assert abs(w[rp[r]:rp[r + 1]].sum() - 1.0) < 1e-12
    # and a dense search at 0.99 keeps strictly more than S1 holds
    dense = np.ones_like(s1)
    rpd, cid, _, _, _ = oracle.block_index(dense)
    g, lse = oracle.block_lse(q, k, rpd, cid, L, b, scale)
    wd = oracle.block_importance(g, lse, rpd, L, b)
    kept = oracle.topp_select(wd, rpd, cid, *dense.shape, 0.99)
    assert kept.sum() > s1.sum()


def test_schedule_selects_on_the_given_weights():
    """With weights supplied for a search step, its Top-p runs on them: one-hot rows
    keep exactly their one block; p = 1 keeps every candidate."""
    q, k, L, b, scale = _static_qk(seed=7)
    H, lp, _ = q.shape
    mb = lp // b
    rp, ci, _, _, _ = oracle.block_index(np.ones((H, mb, mb), dtype=np.uint8))
    onehot = np.zeros(int(rp[-1]), dtype=np.float32)
    hot = {}
    for r in range(H * mb):
        j = (7 * r + 3) % mb
        onehot[rp[r] + j] = 1.0
        hot[r] = j
    _, masks, _ = oracle.gsrs_schedule(3, (1, 2), (0.5, 1.0), lambda t: (q, k), L, b, scale,
                                       w_select={1: onehot})
    m1 = masks[1]
    for r in range(H * mb):
        h, u = divmod(r, mb)
        assert m1[h, u].sum() == 1 and m1[h, u, hot[r]] == 1
    # p = 1 over S1 keeps all of S1
    assert np.array_equal(masks[2], m1)
