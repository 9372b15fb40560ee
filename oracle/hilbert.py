"""Hilbert-curve block organisation (oracle).

The pages' routing front end reorders tokens along a Hilbert curve before
cutting them into blocks, so that tokens that are close in the video (in
time and space) land in the same or nearby blocks (paperlayer.ai summary of
FVAttn, section 3 "FVAttn Design", Sparse-routing frontend).  The pages name
neither the curve construction, nor the axis order, nor what happens on a
grid whose sides are not powers of two.  The reading used here:

* the curve is the 3D Hilbert curve of J. Skilling, "Programming the Hilbert
  curve" (AIP Conf. Proc. 707, 2004), on the smallest cube of side 2^m that
  holds the grid, with the axes in the order (t, y, x);
* grid points outside the T x Y x X box are skipped; the tokens keep the
  curve's order;
* block b is tokens b*B .. b*B + B - 1 of that order (B = 128, the volume of
  the 2x8x8 tiles of the tile layout), so every block is full except the
  last one, which holds the remainder.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def cube_bits(grid) -> int:
    """Smallest m with 2^m >= every side of the grid (at least 1)."""
    side = max(int(g) for g in grid)
    m = 1
    while (1 << m) < side:
        m += 1
    return m


def hilbert_index(coords: np.ndarray, bits: int) -> np.ndarray:
    """Position along the Hilbert curve of each point of a 2^bits cube.

    coords: [P, n] non-negative integers below 2^bits (axis 0 first).
    Returns [P] int64 in [0, 2^(n*bits)).

    Skilling's construction, in two passes over the bit planes from the most
    significant one down: (1) undo the per-level rotations and reflections,
    so that every level of the curve looks like the same Gray-code tour;
    (2) Gray-encode the axes into the "transposed" index, whose bits, read
    plane by plane (axis 0 first within a plane), are the curve position.
    """
    X = np.array(coords, dtype=np.int64, copy=True)
    P, n = X.shape
    top = 1 << (bits - 1)
    # (1) For each level Q (from the top), a point whose axis-i bit is set
    # lies in the "far" half along i: the lower levels of axis 0 are
    # reflected; otherwise axes 0 and i swap their lower bits.
    Q = top
    while Q > 1:
        low = Q - 1
        for i in range(n):
            far = (X[:, i] & Q) != 0
            # reflection of axis 0's lower bits where the point is far
            X[far, 0] ^= low
            # exchange of the lower bits of axes 0 and i where it is near
            near = ~far
            t = (X[near, 0] ^ X[near, i]) & low
            X[near, 0] ^= t
            X[near, i] ^= t
        Q >>= 1
    # (2) Gray encoding: each axis absorbs the one before it, then every
    # axis is corrected by the parity mask taken from the last axis.
    for i in range(1, n):
        X[:, i] ^= X[:, i - 1]
    t = np.zeros(P, dtype=np.int64)
    Q = top
    while Q > 1:
        t ^= np.where((X[:, n - 1] & Q) != 0, Q - 1, 0)
        Q >>= 1
    X ^= t[:, None]
    # interleave: bit plane b (high to low), axis 0 .. n-1
    h = np.zeros(P, dtype=np.int64)
    for b in range(bits - 1, -1, -1):
        for i in range(n):
            h = (h << 1) | ((X[:, i] >> b) & 1)
    return h


def hilbert_token_order(grid) -> np.ndarray:
    """Token indices n = (t*Y + y)*X + x of a T x Y x X grid in Hilbert order."""
    T, Y, X = (int(g) for g in grid)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    coords = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)
    key = hilbert_index(coords, cube_bits(grid))
    return np.argsort(key, kind="stable").astype(np.int64)    # keys are distinct


class HilbertLayout:
    """Blocks = consecutive runs of ``block`` tokens in Hilbert order.

    The same attributes as ``BlockLayout``: ``members[b]`` (the block's tokens
    in curve order), ``sizes``, ``Nb`` and ``N``.
    """

    def __init__(self, grid, block: int = 128):
        self.T, self.Y, self.X = (int(g) for g in grid)
        self.block = int(block)
        assert min(self.T, self.Y, self.X, self.block) >= 1
        self.N = self.T * self.Y * self.X
        self.order = hilbert_token_order(grid)
        self.Nb = -(-self.N // self.block)
        self.members = [self.order[b * self.block:(b + 1) * self.block] for b in range(self.Nb)]
        self.sizes = np.asarray([len(m) for m in self.members], dtype=np.int64)

    @property
    def padded_N(self) -> int:
        return self.Nb * self.block
