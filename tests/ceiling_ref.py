"""Expected outputs of the tile-pattern measurement helper
(mx_ceiling_tile_pattern), recomputed with NumPy from its documented thread
map.  Shared by the GPU test and the CPU test that checks it against a
thread-by-thread emulation."""

import numpy as np


def tile_pattern_expected(x32, rows, cols):
    """Both outputs of the tile-pattern helper from its documented thread
    map, on x viewed as uint32 [rows, cols / 2] (4 words per 16-byte chunk)."""
    row = np.empty((rows, cols // 4), np.uint32)
    row[:, 0::2] = x32[:, 0::4] ^ x32[:, 1::4]
    row[:, 1::2] = x32[:, 2::4] ^ x32[:, 3::4]
    col = np.empty((cols, rows // 4), np.uint32)
    t = np.arange(256)
    w, lane = t >> 6, t & 63
    ch, ry = lane & 15, lane >> 4
    for tr in range(rows // 128):
        for tc in range(cols // 128):
            r0 = tr * 128 + 32 * w + 8 * ry
            for s in range(4):
                q = 256 * s + t
                words = (tc * 128 + 8 * ch) // 2 + np.arange(4)[:, None]          # [4, 256]
                v = x32[r0 + 2 * s, words] ^ x32[r0 + 2 * s + 1, words]
                dst = tr * 32 + 4 * (q & 7) + np.arange(4)[:, None]
                col[tc * 128 + (q >> 3), dst] = v
    return row, col
