"""CPU: the NumPy expectation of the tile-pattern helper equals a literal,
thread-by-thread emulation of the kernel's loads and stores (blocks with
column tiles consecutive, wave w / lane 16 ry + ch reading rows
32 w + 8 ry + i at column 8 ch, then 8 bytes per row and 16-byte column
pieces), so the GPU test compares against what the kernel is meant to do."""

import numpy as np
import pytest

from ceiling_ref import tile_pattern_expected


def emulate(xb, rows, cols):
    row_out = np.zeros(rows * cols, np.uint8)
    col_out = np.zeros(rows * cols, np.uint8)
    n_tc = cols // 128
    for b in range(rows // 128 * n_tc):
        tc, tr = b % n_tc, b // n_tc
        for t in range(256):
            lane, w = t & 63, t >> 6
            ch, ry = lane & 15, lane >> 4
            r0, c0 = tr * 128 + 32 * w + 8 * ry, tc * 128
            v = []
            for i in range(8):
                o = ((r0 + i) * cols + c0 + 8 * ch) * 2
                v.append(xb[o:o + 16].view(np.uint32))
            for i in range(8):
                o = (r0 + i) * cols + c0 + 8 * ch
                row_out[o:o + 8] = np.array([v[i][0] ^ v[i][1], v[i][2] ^ v[i][3]], np.uint32).view(np.uint8)
            for s in range(4):
                q = 256 * s + t
                o = (c0 + (q >> 3)) * rows + tr * 128 + 16 * (q & 7)
                assert o + 16 <= rows * cols
                col_out[o:o + 16] = (v[2 * s] ^ v[2 * s + 1]).view(np.uint8)
    return row_out, col_out


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 256)])
def test_tile_pattern_expectation_matches_emulation(rows, cols):
    xb = np.random.default_rng(rows + cols).integers(0, 256, size=rows * cols * 2, dtype=np.uint8)
    row_out, col_out = emulate(xb, rows, cols)
    row, col = tile_pattern_expected(xb.view(np.uint32).reshape(rows, cols // 2), rows, cols)
    assert np.array_equal(row_out.view(np.uint32).reshape(rows, cols // 4), row)
    assert np.array_equal(col_out.view(np.uint32).reshape(cols, rows // 4), col)
