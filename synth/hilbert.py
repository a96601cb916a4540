"""Locality-preserving token order for video grids.

The GSRS page ("Sparse Attention for Video Generation Acceleration via Growing
Sparsity and Reduced Search", token reordering paragraph) flattens the (t, y, x)
latent grid along a generalized Hilbert curve before blocking, so that each
fixed-size token block holds tokens that are close in space and time.  The page
names the curve by citation only.  The construction restated here is the
recursive generalized Hilbert curve for rectangles of arbitrary size published
by Jakub Cerveny ("gilbert", the generalized Hilbert space-filling curve), in
its three-dimensional form: a box is walked from its origin corner to the far
end of its travel axis; a box much longer along the travel axis than across is
cut into two halves along it; otherwise it is cut into the three legs of a
Hilbert "U" in the plane of the travel axis and the longer of the other two
axes (up the first half, across, back down), the third axis carried through
every leg; halves are kept even where possible so that the legs join with unit
steps.  The code below is this package's own (an explicit stack, cuboids
throughout); the 2-D curve is the same construction on a box one cell deep.
"""

from __future__ import annotations

import numpy as np


def _sign(v: int) -> int:
    return (v > 0) - (v < 0)


def _half(v: int) -> int:
    """v / 2 rounded toward zero (the construction halves signed axis vectors)."""
    return v // 2 if v >= 0 else -((-v) // 2)


def _length(v) -> int:
    return abs(v[0]) + abs(v[1]) + abs(v[2])


def _unit(v):
    return (_sign(v[0]), _sign(v[1]), _sign(v[2]))


def _add(p, *vs):
    return tuple(p[i] + sum(v[i] for v in vs) for i in range(3))


def _scale(v, k: int):
    return (v[0] * k, v[1] * k, v[2] * k)


def _halve(v, even: bool):
    """Half of the axis vector v (toward zero), made even when ``even`` and possible."""
    h = (_half(v[0]), _half(v[1]), _half(v[2]))
    if even and _length(h) % 2 == 1 and _length(v) > 2:
        h = _add(h, _unit(v))
    return h


def gilbert3d(width: int, height: int, depth: int) -> list[tuple[int, int, int]]:
    """All cells (x, y, z) of a width x height x depth box, in curve order.

    Every cell appears once; consecutive cells are face neighbours except for a
    few steps that odd side lengths force (checked by the tests).
    """
    if width <= 0 or height <= 0 or depth <= 0:
        return []
    # A region is (origin, a, b, c): the curve enters at the origin corner and leaves
    # at origin + (|a| - 1) * unit(a); a is the travel axis, b and c span the rest.
    # Each axis vector has exactly one non-zero component.
    axes = sorted([((width, 0, 0), width), ((0, height, 0), height), ((0, 0, depth), depth)],
                  key=lambda t: -t[1])
    stack = [((0, 0, 0), axes[0][0], axes[1][0], axes[2][0])]
    cells: list[tuple[int, int, int]] = []
    while stack:
        o, a, b, c = stack.pop()
        la, lb, lc = _length(a), _length(b), _length(c)
        ua = _unit(a)
        if lb == 1 and lc == 1:  # a line along the travel axis
            cells.extend(_add(o, _scale(ua, i)) for i in range(la))
            continue
        if la == 1:  # a single slab across the travel axis: walk it as a 2-D box
            if lb >= lc:
                stack.append((o, b, c, a))
            else:
                stack.append((o, c, b, a))
            continue
        if 2 * la > 3 * lb and 2 * la > 3 * lc:
            # elongated along the travel axis: two halves one after the other
            a1 = _halve(a, even=True)
            a2 = _add(a, _scale(a1, -1))
            parts = [(o, a1, b, c), (_add(o, a1), a2, b, c)]
        else:
            # Hilbert "U" in the plane of a and the longer of b and c (m); the other
            # axis (n) is carried through every leg
            m, n = (b, c) if lb >= lc else (c, b)
            m1 = _halve(m, even=True)
            m2 = _add(m, _scale(m1, -1))
            a1 = _halve(a, even=False)
            a2 = _add(a, _scale(a1, -1))
            um = _unit(m)
            parts = [
                (o, m1, a1, n),                         # up the first half of m
                (_add(o, m1), a, m2, n),                # across the far half of m
                (_add(o, a, _scale(ua, -1), m1, _scale(um, -1)),
                 _scale(m1, -1), _scale(a2, -1), n),    # back down to the end of a
            ]
        stack.extend(reversed(parts))
    return cells


def gilbert2d(width: int, height: int) -> list[tuple[int, int]]:
    """All cells (x, y) of a width x height rectangle, in curve order."""
    return [(x, y) for (x, y, _) in gilbert3d(width, height, 1)]


def video_hilbert_order(frames: int, height: int, width: int) -> np.ndarray:
    """Permutation of row-major (t, y, x) token ids along the curve over the whole
    (t, y, x) box.  ``order[n]`` is the row-major id of the n-th token on the curve."""
    cells = gilbert3d(width, height, frames)
    return np.array([(t * height + y) * width + x for (x, y, t) in cells], dtype=np.int64)
