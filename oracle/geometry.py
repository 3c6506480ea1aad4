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

Packed edge windows (an alternative reading of the same silence, selected by
``pack_edges``): every full window is still one block, numbered as above
among the full windows; the tokens of all partial windows follow as one
stream, window by window in (frame, window row, window column) order and
row-major inside each window, cut into consecutive blocks of
win_h * win_w tokens. Only the last block can hold fewer tokens; a block of
the stream may mix windows and frames, and pooling is over its tokens like
any other block.
"""

from __future__ import annotations

import numpy as np


class Geometry:
    def __init__(self, frames: int, grid_h: int, grid_w: int, win_h: int, win_w: int, pack_edges: bool = False):
        self.pack_edges = pack_edges
        self.frames = frames
        self.grid_h = grid_h
        self.grid_w = grid_w
        self.win_h = win_h
        self.win_w = win_w
        self.n_wy = -(-grid_h // win_h)
        self.n_wx = -(-grid_w // win_w)
        self.block_size = win_h * win_w
        self.tokens = frames * grid_h * grid_w
        self.n_full = frames * (grid_h // win_h) * (grid_w // win_w)
        if pack_edges:
            edge = self.tokens - self.n_full * self.block_size
            self.n_blocks = self.n_full + -(-edge // self.block_size)
        else:
            self.n_blocks = frames * self.n_wy * self.n_wx

    def windows(self):
        """Token lists (raster indices, row-major) of every window, in
        (frame, window row, window column) order."""
        out = []
        for t in range(self.frames):
            for wy in range(self.n_wy):
                for wx in range(self.n_wx):
                    out.append([(t * self.grid_h + y) * self.grid_w + x
                                for y in range(wy * self.win_h, min((wy + 1) * self.win_h, self.grid_h))
                                for x in range(wx * self.win_w, min((wx + 1) * self.win_w, self.grid_w))])
        return out

    def raster_index(self) -> np.ndarray:
        """[n_blocks, block_size] raster index of each slot's token, -1 if padded."""
        out = np.full((self.n_blocks, self.block_size), -1, dtype=np.int64)
        if self.pack_edges:
            wins = self.windows()
            full = [w for w in wins if len(w) == self.block_size]
            stream = [n for w in wins if len(w) < self.block_size for n in w]
            for b, w in enumerate(full):
                out[b] = w
            for j in range(0, len(stream), self.block_size):
                chunk = stream[j:j + self.block_size]
                out[len(full) + j // self.block_size, :len(chunk)] = chunk
            return out
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
