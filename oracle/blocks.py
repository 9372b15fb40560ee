"""Video-aware block organisation (oracle).

The pages' routing front end groups spatially adjacent tokens into blocks
before routing (FVAttn abstract: blocks organised around the video's layout;
paperlayer.ai summary, section 3 "FVAttn Design", Sparse-routing frontend:
nearby tokens in nearby blocks).  The reading used here: one block is one 3D tile of
(tt, ty, tx) latent tokens, tiles in raster order over the tile grid; an axis
that is not a multiple of its tile size ends in a partial tile, whose missing
tokens simply do not exist (they are never keys and produce no output).
"""
from __future__ import annotations

import numpy as np


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockLayout:
    """Tokens of a T x Y x X grid grouped into tt x ty x tx tiles.

    Token n = (t*Y + y)*X + x.  Block b = (it*nY + iy)*nX + ix.
    ``members[b]`` lists the block's tokens in tile-local raster order.
    """

    def __init__(self, grid, tile):
        self.T, self.Y, self.X = (int(g) for g in grid)
        self.tt, self.ty, self.tx = (int(s) for s in tile)
        assert min(self.T, self.Y, self.X, self.tt, self.ty, self.tx) >= 1
        self.nT = ceil_div(self.T, self.tt)
        self.nY = ceil_div(self.Y, self.ty)
        self.nX = ceil_div(self.X, self.tx)
        self.Nb = self.nT * self.nY * self.nX
        self.N = self.T * self.Y * self.X
        self.members = []
        for it in range(self.nT):
            for iy in range(self.nY):
                for ix in range(self.nX):
                    ts = range(it * self.tt, min(self.T, (it + 1) * self.tt))
                    ys = range(iy * self.ty, min(self.Y, (iy + 1) * self.ty))
                    xs = range(ix * self.tx, min(self.X, (ix + 1) * self.tx))
                    toks = [(t * self.Y + y) * self.X + x for t in ts for y in ys for x in xs]
                    self.members.append(np.asarray(toks, dtype=np.int64))
        self.sizes = np.asarray([len(m) for m in self.members], dtype=np.int64)

    @property
    def padded_N(self) -> int:
        """Tokens after padding every axis up to a tile multiple."""
        return self.nT * self.tt * self.nY * self.ty * self.nX * self.tx
