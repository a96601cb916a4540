"""WaveAlign two-stage query-row reordering, fp64 (test infrastructure only).

Restates WaveAlign §IV (Problem (1), eqs. (2)-(4), Algorithms 1 and 2, the
adaptive skip of §IV-E) step by step.  Readings where the page leaves a step
open:

* Random start block (Algorithm 1): the caller supplies raw start values
  x0 [MB, 2] (drawn by the input generator); they are orthonormalised with the
  same QR rule the iteration uses.
* QR (Algorithm 1): modified Gram-Schmidt with a positive diagonal of R.  If the
  second column vanishes after orthogonalisation (norm <= 1e-12 times the norm
  of the first column, i.e. the centered mask has rank one) the second basis
  vector is set to zero; if the first column is exactly zero both are zero.
* The optional singular-value ordering of Algorithm 1 is applied: the projected
  2 x 2 matrix X^T M~ M~^T X is symmetrised and X is rotated onto its
  eigenvectors in descending eigenvalue order (a library eigensolver here).
* Sign of each basis vector: flipped so that sum_i X[i, k]^3 > 0; when
  |sum| < 1e-6 the first entry with magnitude > 1e-6 is made positive instead.
  (The page calls the angular order invariant to sign flips; a flip in fact
  reverses or rotates the circular order, so a fixed convention is needed for
  the result to be a function of the mask and x0 alone.)
* Angle (eq. (4)): a_i = atan2(u2[i], u1[i]); negative values get 2*pi added,
  -0.0 becomes +0.0; ascending order as in the Fig. 6 example; ties keep the
  lower row index (stable sort).
* A mask whose rows are all identical has a zero centered mask; Stage 1 then
  keeps the identity order (no subspace exists to embed into).
* Waves: the ordered rows are cut into ``n_slices`` contiguous slices of
  ceil(MB / n_slices) positions (one per cache domain), and each slice into
  consecutive buckets of at most W positions, the last one short.
  ``n_slices = 1`` is Algorithm 2 exactly.
* Stage 2 (§IV-D): within a bucket rows are sorted by descending NNZ; equal NNZ
  keep their Stage-1 order (as rows r0, r2, r7 and r5, r6 do in Fig. 7(b)).
* Adaptive skip (§IV-E names three cases and offline profiles, no formula):
  reorder a head only if (i) its K/V working set NB*b*d*2 bytes * 2 exceeds
  ``ws_min_bytes`` (the K/V set does not fit the cache), (ii) the selected work
  4*b*b*d*nnz FLOP of the heaviest head reordered in the same call is at least
  ``flops_min`` (enough work to amortise the reorder), and (iii) the pooled
  Jaccard similarity of adjacent rows, sum_u |R_u & R_u+1| / sum_u |R_u | R_u+1|,
  is below ``jaccard_max`` (rows are not already local).  An empty pooled union
  counts as similarity 1.  The work case is read per call rather than per head:
  the heads of one call are reordered side by side, so the call costs what its
  slowest head costs, and once one head's work pays for it the other heads are
  reordered at no extra cost.  With a single head the two readings agree.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TWO_PI = 2.0 * np.pi

SKIP_ADAPTIVE = 0
SKIP_NEVER = 1
SKIP_ALWAYS = 2


@dataclass
class ReorderParams:
    wave: int = 64             # W: rows per wave bucket
    n_slices: int = 8          # contiguous slices of the order (1 = Algorithm 2 as printed)
    iters: int = 10            # T of Algorithm 1
    stage1: bool = True
    stage2: bool = True
    skip_mode: int = SKIP_ADAPTIVE
    ws_min_bytes: float = 0.0
    flops_min: float = 0.0
    jaccard_max: float = 1.0


def centered_mask(mask_h: np.ndarray) -> np.ndarray:
    """WaveAlign eq. (2): M~ = (I - 11^T/MB) M (the mean row subtracted from every row)."""
    m = np.asarray(mask_h, dtype=np.float64)
    return m - m.mean(axis=0, keepdims=True)


def _qr2(z: np.ndarray) -> np.ndarray:
    """Q factor of an MB x 2 block by modified Gram-Schmidt (positive diag of R)."""
    q = np.zeros_like(z)
    n1 = np.sqrt(z[:, 0] @ z[:, 0])
    if n1 == 0.0:
        return q
    q[:, 0] = z[:, 0] / n1
    r12 = q[:, 0] @ z[:, 1]
    w = z[:, 1] - r12 * q[:, 0]
    n2 = np.sqrt(w @ w)
    if n2 > 1e-12 * n1:
        q[:, 1] = w / n2
    return q


def canonical_signs(x: np.ndarray) -> np.ndarray:
    x = np.array(x, dtype=np.float64, copy=True)
    for kk in range(x.shape[1]):
        s = np.sum(x[:, kk] * x[:, kk] * x[:, kk])
        if abs(s) >= 1e-6:
            flip = s < 0.0
        else:
            big = np.flatnonzero(np.abs(x[:, kk]) > 1e-6)
            flip = big.size > 0 and x[big[0], kk] < 0.0
        if flip:
            x[:, kk] = -x[:, kk]
    return x


def mfcsi(mask_h: np.ndarray, x0: np.ndarray, iters: int, ritz: bool = True):
    """Rank-2 spectral embedding of the mask rows (WaveAlign §IV-C-2, Algorithm 1).

    The embedding of row i is row i of the two leading left singular vectors of the
    centered mask M~ (eq. (2)), which are the two leading eigenvectors of the row
    Gram matrix M~ M~^T.  They are approximated by subspace iteration from the start
    block x0: X <- qr(M~ (M~^T X)), ``iters`` times, with M~ formed explicitly in
    fp64.  With ``ritz`` the two basis vectors are then rotated onto the eigenvectors
    of the projected 2 x 2 matrix X^T M~ M~^T X, in descending eigenvalue order.  The
    sign convention of ``canonical_signs`` fixes the result.  Returns None when every
    row of the mask is the same (M~ = 0: there is no subspace to embed into).
    """
    mt = centered_mask(mask_h)                 # M~, MB x NB
    if not np.any(mt):
        return None

    def gram_times(xx):                        # M~ M~^T X, never forming the MB x MB Gram
        return mt @ (mt.T @ xx)

    x = _qr2(np.asarray(x0, dtype=np.float64))
    for _ in range(iters):
        x = _qr2(gram_times(x))
    if ritz:
        proj = x.T @ gram_times(x)
        proj = 0.5 * (proj + proj.T)
        _, vecs = np.linalg.eigh(proj)         # ascending eigenvalues
        x = x @ vecs[:, ::-1]
    return canonical_signs(x)


def polar_angles(u: np.ndarray) -> np.ndarray:
    """WaveAlign eq. (4), mapped to [0, 2*pi] as the Fig. 6 angles are."""
    a = np.arctan2(u[:, 1], u[:, 0])
    a = np.where(a < 0.0, a + TWO_PI, a)
    return a + 0.0


def stage1_order(angles: np.ndarray) -> np.ndarray:
    """Rows sorted by ascending angle, ties by row index."""
    return np.argsort(angles, kind="stable")


def wave_buckets(mb: int, n_slices: int, wave: int):
    """Position ranges [lo, hi) of the wave buckets, slice by slice."""
    s = -(-mb // n_slices)
    out = []
    for x in range(n_slices):
        lo, hi = x * s, min((x + 1) * s, mb)
        for b in range(lo, hi, wave):
            out.append((b, min(b + wave, hi)))
    return out


def stage2_order(order: np.ndarray, nnz: np.ndarray, buckets) -> np.ndarray:
    """WaveAlign §IV-D: descending NNZ inside each bucket, stable."""
    perm = np.array(order, dtype=np.int64, copy=True)
    for lo, hi in buckets:
        rows = perm[lo:hi]
        perm[lo:hi] = rows[np.argsort(-nnz[rows], kind="stable")]
    return perm


def skip_statistics(mask_h: np.ndarray, block: int, head_dim: int) -> np.ndarray:
    """[nnz, density, K/V working-set bytes, selected FLOP, adjacent-row Jaccard]."""
    m = np.asarray(mask_h).astype(bool)
    mb, nb = m.shape
    nnz = int(m.sum())
    inter = int(np.sum(m[:-1] & m[1:]))
    union = int(np.sum(m[:-1] | m[1:]))
    jac = 1.0 if union == 0 else float(inter) / float(union)
    ws = float(nb * block * head_dim * 2 * 2)
    flops = 4.0 * block * block * head_dim * nnz
    return np.array([float(nnz), nnz / float(mb * nb), ws, flops, jac])


def skip_decision(stats: np.ndarray, p: ReorderParams, call_flops: float | None = None) -> bool:
    """True if the head keeps its original order.  ``call_flops`` is the selected
    FLOP of the heaviest head of the call (the head's own, stats[3], by default)."""
    if p.skip_mode == SKIP_ALWAYS:
        return True
    if p.skip_mode == SKIP_NEVER:
        return False
    work = stats[3] if call_flops is None else call_flops
    reorder = stats[2] > p.ws_min_bytes and work >= p.flops_min and stats[4] < p.jaccard_max
    return not reorder


def reorder_head(mask_h: np.ndarray, x0_h: np.ndarray, block: int, head_dim: int,
                 p: ReorderParams, call_flops: float | None = None):
    """WaveAlign Algorithm 2 for one head (``call_flops``: as in skip_decision).

    Returns (perm, skipped, angles, stats); ``perm[pos]`` is the query block run
    at position ``pos``; angles are NaN where Stage 1 did not run.
    """
    mb = mask_h.shape[0]
    nnz = np.asarray(mask_h).astype(np.int64).sum(axis=1)
    stats = skip_statistics(mask_h, block, head_dim)
    angles = np.full(mb, np.nan)
    if skip_decision(stats, p, call_flops):
        return np.arange(mb, dtype=np.int64), True, angles, stats
    order = np.arange(mb, dtype=np.int64)
    if p.stage1:
        u = mfcsi(mask_h, x0_h, p.iters)
        if u is not None:
            angles = polar_angles(u)
            order = stage1_order(angles)
    perm = order
    if p.stage2:
        perm = stage2_order(order, nnz, wave_buckets(mb, p.n_slices, p.wave))
    return perm, False, angles, stats


def reorder_rows(mask: np.ndarray, x0: np.ndarray, block: int, head_dim: int,
                 p: ReorderParams):
    """All heads: (perm [H, MB], inv_perm [H, MB], skipped [H], angles [H, MB], stats [H, 5])."""
    H, mb, _ = mask.shape
    perm = np.zeros((H, mb), dtype=np.int64)
    inv = np.zeros((H, mb), dtype=np.int64)
    skipped = np.zeros(H, dtype=bool)
    angles = np.full((H, mb), np.nan)
    stats = np.zeros((H, 5))
    # the work case of the adaptive skip looks at the heaviest head of the call
    call_flops = max(4.0 * block * block * head_dim * float(np.count_nonzero(mask[h]))
                     for h in range(H))
    for h in range(H):
        perm[h], skipped[h], angles[h], stats[h] = reorder_head(mask[h], x0[h], block, head_dim, p,
                                                                call_flops)
        inv[h, perm[h]] = np.arange(mb)
    return perm, inv, skipped, angles, stats
