"""GPU: the measurement helpers behind the benchmark's roofline fractions.
The streaming copy reproduces its source byte for byte (so its rate is a
real read + write rate), the tile-pattern helper writes exactly the bytes
its thread map defines and nothing past its outputs (so it moves the
traffic it claims), and the MFMA loop writes finite sums."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
from ceiling_ref import tile_pattern_expected

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [4096, 3 * 4096, 1 << 22])
def test_ceiling_copy_is_exact(nbytes):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 4096,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.full_like(src, 0xA5)
    mxa.mx_ceiling_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool((dst[nbytes:] == 0xA5).all())        # nothing written past the end


def test_ceiling_mfma_writes_finite_sums():
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    for rnd in (True, False):
        mxa.mx_ceiling_mfma(out, 4, 3, rnd)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (384, 256)])
def test_ceiling_tile_pattern_moves_the_documented_bytes(rows, cols):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(rows * 7 + cols)
    x = torch.randint(-2**31, 2**31 - 1, (rows, cols // 2), dtype=torch.int32, device="cuda:0", generator=g)
    row_out = torch.full((rows * cols + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
    col_out = torch.full((rows * cols + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
    mxa.mx_ceiling_tile_pattern(x, row_out, col_out, rows, cols)
    torch.cuda.synchronize()
    row, col = tile_pattern_expected(x.cpu().numpy().view(np.uint32), rows, cols)
    assert np.array_equal(row_out[:rows * cols].cpu().numpy().view(np.uint32).reshape(rows, cols // 4), row)
    assert np.array_equal(col_out[:rows * cols].cpu().numpy().view(np.uint32).reshape(cols, rows // 4), col)
    for buf in (row_out, col_out):
        assert bool((buf[rows * cols:] == 0xA5).all())   # nothing written past the end
