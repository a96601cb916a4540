"""Locality-preserving token order for video grids.

The GSRS page ("Sparse Attention for Video Generation Acceleration via Growing
Sparsity and Reduced Search", token reordering paragraph) flattens the (t, y, x)
latent grid along a generalized Hilbert curve before blocking, so that each
fixed-size token block holds spatially adjacent tokens.  The page names the
curve by citation only.  The reading taken here: inside every frame the tokens
follow a generalized Hilbert curve over the (y, x) rectangle, written below from
the published recursive construction for arbitrary rectangles (split the long
side in two when the rectangle is elongated, otherwise lay out the three legs of
a Hilbert "U"); consecutive frames run the curve forwards and backwards in
turn, so the step from one frame to the next is a unit step in t.
"""

from __future__ import annotations

import numpy as np


def _sign(v: int) -> int:
    return (v > 0) - (v < 0)


def _half(v: int) -> int:
    """v / 2 rounded toward zero (the construction halves signed axis vectors)."""
    return v // 2 if v >= 0 else -((-v) // 2)


def gilbert2d(width: int, height: int) -> list[tuple[int, int]]:
    """All cells (x, y) of a width x height rectangle, in curve order.

    Every cell appears once.  Consecutive cells are 4-neighbours except for at
    most a few diagonal steps that odd side lengths force.
    """
    if width <= 0 or height <= 0:
        return []
    cells: list[tuple[int, int]] = []
    # A region is (x, y, ax, ay, bx, by): start corner, major axis vector a
    # (walked first) and minor axis vector b; exactly one component of each
    # vector is non-zero.  Regions are processed depth-first, in order.
    if width >= height:
        stack = [(0, 0, width, 0, 0, height)]
    else:
        stack = [(0, 0, 0, height, width, 0)]
    while stack:
        x, y, ax, ay, bx, by = stack.pop()
        la = abs(ax + ay)
        lb = abs(bx + by)
        ux, uy = _sign(ax), _sign(ay)
        vx, vy = _sign(bx), _sign(by)
        if lb == 1:  # a single line along the major axis
            for i in range(la):
                cells.append((x + i * ux, y + i * uy))
            continue
        if la == 1:  # a single line along the minor axis
            for i in range(lb):
                cells.append((x + i * vx, y + i * vy))
            continue
        hax, hay = _half(ax), _half(ay)
        hbx, hby = _half(bx), _half(by)
        if 2 * la > 3 * lb:
            # Elongated: two halves side by side along the major axis.  Keep the
            # first half even so that the curve can return to its side.
            if abs(hax + hay) % 2 == 1 and la > 2:
                hax, hay = hax + ux, hay + uy
            parts = [
                (x, y, hax, hay, bx, by),
                (x + hax, y + hay, ax - hax, ay - hay, bx, by),
            ]
        else:
            # Hilbert "U": up the first half of the minor axis, across the full
            # major axis, back down the other side.
            if abs(hbx + hby) % 2 == 1 and lb > 2:
                hbx, hby = hbx + vx, hby + vy
            parts = [
                (x, y, hbx, hby, hax, hay),
                (x + hbx, y + hby, ax, ay, bx - hbx, by - hby),
                (x + (ax - ux) + (hbx - vx), y + (ay - uy) + (hby - vy),
                 -hbx, -hby, -(ax - hax), -(ay - hay)),
            ]
        stack.extend(reversed(parts))
    return cells


def video_hilbert_order(frames: int, height: int, width: int) -> np.ndarray:
    """Permutation of row-major (t, y, x) token ids along the frame-wise curve.

    ``order[n]`` is the row-major id of the n-th token on the curve.
    """
    plane = gilbert2d(width, height)
    ids = np.array([y * width + x for (x, y) in plane], dtype=np.int64)
    out = np.empty(frames * height * width, dtype=np.int64)
    per = height * width
    for t in range(frames):
        seq = ids if t % 2 == 0 else ids[::-1]
        out[t * per:(t + 1) * per] = t * per + seq
    return out
