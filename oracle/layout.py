"""Tile map of the multi-view token sequence (oracle side).

Source: Zebra3D pages, "Linear-centered stages plus tile-sparse stages":
each image is cut into tiles of 8x8 patches, 64 tokens for a complete tile
(the Chinese page stresses *complete* tiles, so edge tiles can be partial).

Readings (the pages fix none of these):
  * token order inside a frame: the S special tokens first, then the patch
    grid in row-major order;
  * tile numbering: frame-major, then tile row, then tile column; this order
    defines "lower tile index" for tie-breaks;
  * tokens inside a tile are listed row-major.
"""
from __future__ import annotations

import numpy as np


class TileMap:
    """Tiles of an (F, S, R, C) multi-view sequence.

    Attributes
      N            number of tokens, F*(S + R*C)
      T            number of tiles, F*ceil(R/8)*ceil(C/8)
      tokens[u]    int64 array of the token indices in tile u (row-major)
      n[u]         tile size
      specials     int64 array of all special-token indices (frame order)
      tile_of      int64 [N]: tile of each patch token, -1 for specials
    """

    def __init__(self, frames: int, specials: int, rows: int, cols: int):
        self.F, self.S, self.R, self.C = frames, specials, rows, cols
        self.tpf = specials + rows * cols
        self.N = frames * self.tpf
        tr = (rows + 7) // 8
        tc = (cols + 7) // 8
        self.tiles_per_frame = tr * tc
        self.T = frames * tr * tc
        self.tokens = []
        self.tile_of = np.full(self.N, -1, dtype=np.int64)
        for f in range(frames):
            base = f * self.tpf + specials
            for a in range(tr):
                for b in range(tc):
                    toks = [base + r * cols + c
                            for r in range(8 * a, min(8 * a + 8, rows))
                            for c in range(8 * b, min(8 * b + 8, cols))]
                    u = len(self.tokens)
                    arr = np.array(toks, dtype=np.int64)
                    self.tokens.append(arr)
                    self.tile_of[arr] = u
        self.n = np.array([len(t) for t in self.tokens], dtype=np.int64)
        self.specials = np.array([f * self.tpf + s for f in range(frames)
                                  for s in range(specials)], dtype=np.int64)

    def is_special(self, token: int) -> bool:
        return self.tile_of[token] < 0

    def patch_position(self, token: int):
        """(row, col) of a patch token; specials return None."""
        loc = token % self.tpf
        if loc < self.S:
            return None
        p = loc - self.S
        return p // self.C, p % self.C


def keep_count(y: float, T: int) -> int:
    """Number of key tiles kept per query tile.

    Source: "Linear-centered stages plus tile-sparse stages" -- the selector
    keeps a key-tile fraction of 1 - y. Reading: round to nearest with ties
    to even (Python's round on a float), clamped to [0, T]. Floor would
    give 159 instead of 160 at T = 800, y = 0.8, because (1 - 0.8) * 800 is
    159.99999999999997 in double.
    """
    if not (0.0 <= y <= 1.0):
        raise ValueError("y must lie in [0, 1]")
    return max(0, min(T, int(round((1.0 - y) * T))))
