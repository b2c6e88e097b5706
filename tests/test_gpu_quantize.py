"""GPU parity: MXFP8 quantize / dequantize kernels vs the oracle, bit-exact
(OCP MX rules; digest "Key Questions Answered"; pytorch/ao PR #3203 quantize
and dequantize kernels)."""

import json
import os
import struct

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from oracle import mxfp8 as mx

from gpu_util import dev, host, spanels, srows

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_quant(xb, rowwise=True, colwise=False, rows_out=None, gather=None, batch=None):
    x = dev(xb)
    if batch is not None:
        x = x.view(batch, -1, xb.shape[-1])
    g = dev(np.asarray(gather, np.int32)) if gather is not None else None
    q, s, qt, st = mxa.quantize(x, rowwise=rowwise, colwise=colwise, rows_out=rows_out, gather=g)
    torch.cuda.synchronize()
    nb = 1 if batch is None else batch
    cols = xb.shape[-1]
    ro = x.shape[-2] if rows_out is None else rows_out
    out = [None] * 4
    if q is not None:   # scales back to [.., rows, cols/32] (pad bytes checked zero)
        out[0] = host(q)
        out[1] = srows(s, cols).reshape(q.shape[:-1] + (cols // 32,))
    if qt is not None:
        out[2] = host(qt)
        out[3] = srows(st, ro).reshape(qt.shape[:-1] + (ro // 32,))
        assert st.shape[1] == nb * cols
    return out


def test_golden_blocks():
    with open(os.path.join(GOLDEN, "quant_blocks.json")) as fh:
        blocks = json.load(fh)["blocks"]
    rows, wq, ws = [], [], []
    for b in blocks:
        if "values" in b:
            rows.append([struct.unpack("<I", struct.pack("<f", v))[0] >> 16 for v in b["values"]])
        else:
            rows.append([int(h, 16) for h in b["bf16_bits"]])
        wq.append([int(h, 16) for h in b["codes"]])
        ws.append(b["scale_byte"])
    xb = np.array(rows, np.uint16)
    q, s, _, _ = gpu_quant(xb)
    assert np.array_equal(q, np.array(wq, np.uint8)) and np.array_equal(s[:, 0], np.array(ws, np.uint8))


def exhaustive_blocks():
    """Blocks that put every finite bf16 pattern (both signs) under every
    reachable scale byte: element 0 fixes the block amax (exponent field
    byte + 8, largest mantissa), elements 1..31 run through all patterns whose
    magnitude does not exceed it."""
    blocks = []
    for sb in range(0, 247):
        E = max(sb + 8, 8)
        amax = (E << 7) | 0x7F
        mags = np.arange(0, amax + 1, dtype=np.uint32)
        pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-pats.size // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:pats.size] = pats
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = amax
        blk[:, 1:] = body.reshape(n, 31)
        blocks.append(blk)
    b = np.concatenate(blocks)
    pad = -b.shape[0] % 64
    b = np.concatenate([b, np.zeros((pad, 32), np.uint16)])
    return b.reshape(-1, 64 * 32)


def test_rowwise_exhaustive_patterns_and_scales():
    xb = exhaustive_blocks()
    R = xb.shape[0]
    q, s, qt, st = gpu_quant(xb, rowwise=True, colwise=True, rows_out=-(-R // 32) * 32)
    oq, os_ = mx.quantize_rowwise(xb)
    assert np.array_equal(s[:R], os_)
    assert np.array_equal(q[:R], oq)
    assert np.all(q[R:] == 0) and np.all(s[R:] == 0)        # rows past the source are zero rows
    cq, cs = mx.quantize_colwise(xb, rows_out=qt.shape[1])
    assert np.array_equal(st, cs) and np.array_equal(qt, cq)


def test_fused_rowcol_workload4_slice():
    xb = workloads.quant_tensor(4, 4096, 5120, chunk=1)
    q, s, qt, st = gpu_quant(xb, rowwise=True, colwise=True)
    oq, os_ = mx.quantize_rowwise(xb)
    assert np.array_equal(s, os_) and np.array_equal(q, oq)
    cq, cs = mx.quantize_colwise(xb)
    assert np.array_equal(st, cs) and np.array_equal(qt, cq)
    # dequantize both orientations back to bf16
    y = host(mxa.dequantize(dev(q), dev(spanels(s))))
    assert np.array_equal(y, mx.dequantize(oq, os_))
    yt = host(mxa.dequantize(dev(qt), dev(spanels(st))))
    assert np.array_equal(yt, mx.dequantize(cq, cs))


def test_workload4_full_size_sampled():
    """[16*8192, 5120] with zero, subnormal and outlier tiles; fused row+col
    quantize and both dequantizes at full size, checked on sampled rows and
    columns (the oracle computes those one by one)."""
    xb = workloads.quant_tensor(4, 131072, 5120)
    x = dev(xb)
    q, s, qt, st = mxa.quantize(x, rowwise=True, colwise=True)
    y = mxa.dequantize(q, s)
    yt = mxa.dequantize(qt, st)
    torch.cuda.synchronize()
    g = np.random.default_rng(44)
    rows = np.sort(g.choice(131072, 256, replace=False))
    cols = np.sort(g.choice(5120, 24, replace=False))
    ridx = torch.from_numpy(rows).to(x.device)
    cidx = torch.from_numpy(cols).to(x.device)
    oq, os_ = mx.quantize_rowwise(xb[rows])
    assert np.array_equal(host(q[ridx]), oq) and np.array_equal(srows(s[:, ridx], 5120), os_)
    assert np.array_equal(host(y[ridx]), mx.dequantize(oq, os_))
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(xb[:, cols].T))
    assert np.array_equal(host(qt[cidx]), cq) and np.array_equal(srows(st[:, cidx], 131072), cs)
    assert np.array_equal(host(yt[cidx]), mx.dequantize(cq, cs))


def test_colwise_gather_padding_and_batch():
    g = np.random.default_rng(12)
    xb = workloads.normal_bf16(g, (200, 96), outlier_p=0.01)
    gather = g.integers(-1, 200, 256)
    gather[:5] = [-1, 199, 199, 0, 1000]   # zero row, duplicate, out-of-range -> zero row
    q, s, qt, st = gpu_quant(xb, rowwise=True, colwise=True, rows_out=256, gather=gather)
    safe = np.where(gather < 200, gather, -1)
    oq, os_ = mx.quantize_rowwise(mx.gather_rows(xb, safe, 256))
    assert np.array_equal(q, oq) and np.array_equal(s, os_)
    cq, cs = mx.quantize_colwise(xb, rows_out=256, gather=safe)
    assert np.array_equal(qt, cq) and np.array_equal(st, cs)
    # colwise only, no gather, rows_out > rows (zero tail rows)
    _, _, qt2, st2 = gpu_quant(xb, rowwise=False, colwise=True, rows_out=224)
    cq2, cs2 = mx.quantize_colwise(xb, rows_out=224)
    assert np.array_equal(qt2, cq2) and np.array_equal(st2, cs2)
    # batched weights [E, N, K]: rowwise along K and columnwise along N per expert
    w = np.stack([workloads.normal_bf16(g, (96, 64), 0.02) for _ in range(3)])
    q, s, qt, st = gpu_quant(w.reshape(-1, 64), rowwise=True, colwise=True, batch=3)
    for e in range(3):
        oq, os_ = mx.quantize_rowwise(w[e])
        cq, cs = mx.quantize_colwise(w[e])
        assert np.array_equal(q[e], oq) and np.array_equal(s[e], os_)
        assert np.array_equal(qt[e], cq) and np.array_equal(st[e], cs)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 64), (5, 544), (33, 32), (7, 2080)])
def test_rowwise_ragged_shapes(rows, cols):
    g = np.random.default_rng(rows * 1000 + cols)
    xb = workloads.normal_bf16(g, (rows, cols), outlier_p=0.05)
    q, s, _, _ = gpu_quant(xb)
    oq, os_ = mx.quantize_rowwise(xb)
    assert np.array_equal(q, oq) and np.array_equal(s, os_)


def test_dequantize_exhaustive_codes_and_scales():
    c, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    q = np.repeat(c.reshape(-1, 1).astype(np.uint8), 32, axis=1)
    s = b.reshape(-1, 1).astype(np.uint8)
    y = host(mxa.dequantize(dev(q), dev(spanels(s))))
    ref = mx.dequantize(q, s)
    nan = np.isnan(mx.bf16_to_f64(ref))
    assert np.array_equal(np.isnan(mx.bf16_to_f64(y)), nan)
    assert np.array_equal(y[~nan], ref[~nan])


def test_quantize_deterministic():
    xb = workloads.quant_tensor(4, 1024, 2048, chunk=2)
    a = gpu_quant(xb, rowwise=True, colwise=True)
    b = gpu_quant(xb, rowwise=True, colwise=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
