"""Token geometry: raster tokens <-> (block, slot) of per-frame 2D windows.

[DA1] abstract and [DA1-article] steps 1 and 4: every frame's latent map is
split into 2D spatial windows (8x16 in the article); queries, keys and values
are reordered so that each window's tokens are contiguous, and the original
order is restored after attention. [DA2] abstract: pooling is spatial 2D per
frame.

Readings (the pages are silent on them):
* A frame whose grid is not a multiple of the window is padded up to whole
  windows, so every block is exactly one window; padded slots hold no token.
  Every window keeps at least one real token because the window count is the
  ceiling of grid / window.
* Windows are numbered (frame, window row, window column), row-major; slots
  inside a window are (row, column), row-major.
"""

from __future__ import annotations

import numpy as np


class Geometry:
    def __init__(self, frames: int, grid_h: int, grid_w: int, win_h: int, win_w: int):
        self.frames = frames
        self.grid_h = grid_h
        self.grid_w = grid_w
        self.win_h = win_h
        self.win_w = win_w
        self.n_wy = -(-grid_h // win_h)
        self.n_wx = -(-grid_w // win_w)
        self.n_blocks = frames * self.n_wy * self.n_wx
        self.block_size = win_h * win_w
        self.tokens = frames * grid_h * grid_w

    def raster_index(self) -> np.ndarray:
        """[n_blocks, block_size] raster index of each slot's token, -1 if padded."""
        out = np.full((self.n_blocks, self.block_size), -1, dtype=np.int64)
        for t in range(self.frames):
            for wy in range(self.n_wy):
                for wx in range(self.n_wx):
                    b = (t * self.n_wy + wy) * self.n_wx + wx
                    for iy in range(self.win_h):
                        for ix in range(self.win_w):
                            y = wy * self.win_h + iy
                            x = wx * self.win_w + ix
                            if y < self.grid_h and x < self.grid_w:
                                out[b, iy * self.win_w + ix] = (t * self.grid_h + y) * self.grid_w + x
        return out


def gather_blocks(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """x [N, d] -> [n_blocks, block_size, d], padded slots zero."""
    out = np.zeros(idx.shape + (x.shape[1],), dtype=x.dtype)
    valid = idx >= 0
    out[valid] = x[idx[valid]]
    return out
