"""GPU parity: the SwiGLU and combine glue of the expert FFN, with their fused
requantize, vs the oracle (oracle/glue.py, oracle/mxfp8.py).

* bf16 results (A, dH, the combine output) pass the element-wise glue rule
  of oracle/tolerance.py against the exact fp64 values;
* the combine backward's bf16 values are bit-exact (one fp32 product, one
  RNE rounding on both sides);
* every MX code and scale byte is bit-exact against the oracle's quantize of
  the bf16 values the kernel produced (the requantize is checked stage-wise
  on the kernel's own bf16 results, which the same call writes out).
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from oracle import glue
from oracle import mxfp8 as mx
from oracle import routing, tolerance

from gpu_util import dev, host, srows

pytestmark = pytest.mark.gpu


def check_mx(vals_bits, rq, rs, cq, cs):
    """Row and column MX outputs equal the oracle's quantize of vals_bits."""
    R, C = vals_bits.shape
    if rq is not None:
        oq, os_ = mx.quantize_rowwise(vals_bits)
        assert np.array_equal(host(rq), oq)
        assert np.array_equal(srows(rs, C), os_)
    if cq is not None:
        oq, os_ = mx.quantize_colwise(vals_bits)
        assert np.array_equal(host(cq), oq)
        assert np.array_equal(srows(cs, R), os_)


def h_input(g, rows, F, pad_rows=()):
    """H [rows, 2F]: N(0, 2) with outliers, a few huge and tiny magnitudes;
    pad rows zero."""
    h = workloads.normal_bf16(g, (rows, 2 * F), 2.0, outlier_p=0.002)
    special = mx.f64_to_bf16(np.array([-1e30, 1e30, -200.0, 200.0, 1e-40, -1e-40, 0.0, -0.0, -1.2785]))
    idx = g.integers(0, h.size, special.size * 4)
    h.ravel()[idx] = np.tile(special, 4)
    h[list(pad_rows)] = 0
    return h


@pytest.mark.parametrize("rows,F", [(256, 128), (224, 96), (96, 2048), (1056, 160), (32, 32)])
def test_swiglu_fwd(rows, F):
    g = np.random.default_rng(rows + F)
    h = h_input(g, rows, F, pad_rows=range(rows - 7, rows))
    a, rq, rs, cq, cs = mxa.swiglu_quantize(dev(h), rowwise=True, colwise=True, want_bf16=True)
    torch.cuda.synchronize()
    ab = host(a)
    exact, S = glue.swiglu(h, F)
    res = tolerance.check_bf16_elementwise(ab, exact, S)
    print("swiglu", res)
    assert res["ok"], res
    assert np.all(ab[rows - 7:] == 0)
    check_mx(ab, rq, rs, cq, cs)
    # the MX results do not depend on whether A itself is written
    _, rq2, rs2, cq2, cs2 = mxa.swiglu_quantize(dev(h), rowwise=True, colwise=True, want_bf16=False)
    torch.cuda.synchronize()
    for u, v in ((rq, rq2), (rs, rs2), (cq, cq2), (cs, cs2)):
        assert torch.equal(u, v)


def test_swiglu_rowwise_only_ragged_rows():
    g = np.random.default_rng(7)
    h = h_input(g, 45, 64)
    a, rq, rs, cq, cs = mxa.swiglu_quantize(dev(h), rowwise=True, colwise=False, want_bf16=True)
    torch.cuda.synchronize()
    assert cq is None
    ab = host(a)
    exact, S = glue.swiglu(h, 64)
    assert tolerance.check_bf16_elementwise(ab, exact, S)["ok"]
    check_mx(ab, rq, rs, None, None)


@pytest.mark.parametrize("rows,F", [(256, 128), (224, 96), (160, 2048), (32, 32)])
def test_swiglu_bwd(rows, F):
    g = np.random.default_rng(3 * rows + F)
    h = h_input(g, rows, F, pad_rows=range(5))
    da = workloads.normal_bf16(g, (rows, F), 1.0, outlier_p=0.002)
    da[:5] = 0
    dh, rq, rs, cq, cs = mxa.swiglu_bwd_quantize(dev(h), dev(da), rowwise=True, colwise=True, want_bf16=True)
    torch.cuda.synchronize()
    dhb = host(dh)
    exact, S = glue.swiglu_bwd(h, da, F)
    res = tolerance.check_bf16_elementwise(dhb, exact, S)
    print("swiglu_bwd", res)
    assert res["ok"], res
    assert np.all(dhb[:5] == 0) or np.all(mx.bf16_to_f64(dhb[:5]) == 0)
    check_mx(dhb, rq, rs, cq, cs)
    _, rq2, rs2, cq2, cs2 = mxa.swiglu_bwd_quantize(dev(h), dev(da), rowwise=True, colwise=True, want_bf16=False)
    torch.cuda.synchronize()
    for u, v in ((rq, rq2), (rs, rs2), (cq, cq2), (cs, cs2)):
        assert torch.equal(u, v)


def routed(g, T, E, topk, dup=False):
    if dup:
        ids = g.integers(0, E, (T, topk))
    else:
        ids = np.stack([g.permutation(E)[:topk] for _ in range(T)])
    logits = g.standard_normal((T, topk)).astype(np.float32)
    w = np.exp(logits - logits.max(1, keepdims=True))
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    counts, off, dst, src = routing.route(ids, E, workloads.capacity(T, topk, E))
    return ids, w, off, dst, src


@pytest.mark.parametrize("T,H,E,topk,dup", [(300, 96, 6, 2, False), (128, 2048, 16, 8, False),
                                            (77, 544, 4, 3, True), (64, 32, 3, 1, False), (40, 160, 64, 9, False),
                                            (50, 96, 128, 64, False)])   # top-64, the router's largest k
def test_combine(T, H, E, topk, dup):
    g = np.random.default_rng(T * H + topk)
    ids, w, off, dst, src = routed(g, T, E, topk, dup)
    rows = src.size
    y = workloads.normal_bf16(g, (rows, H), 1.0, outlier_p=0.01)
    out = host(mxa.combine(dev(y), dev(dst), dev(w), T, topk))
    exact, S = glue.combine(y, dst, w, topk)
    # k fused multiply-adds in j order: at most k fp32 roundings of the
    # magnitude sum (the default glue bound covers k <= 8)
    rel = max(tolerance.GLUE_REL, 2.0 * topk * 2.0 ** -24)
    res = tolerance.check_bf16_elementwise(out, exact, S, rel)
    print("combine", res)
    assert res["ok"], res
    # unweighted: the backward of the permute
    out1 = host(mxa.combine(dev(y), dev(dst), None, T, topk))
    exact1, S1 = glue.combine(y, dst, None, topk)
    assert tolerance.check_bf16_elementwise(out1, exact1, S1, rel)["ok"]


def test_combine_top1_unit_weight_is_exact_unpermute():
    g = np.random.default_rng(11)
    T, H, E = 500, 256, 7
    ids = g.integers(0, E, (T, 1))
    _, off, dst, src = routing.route(ids, E)
    x = workloads.normal_bf16(g, (T, H), outlier_p=0.01)
    xp = np.zeros((src.size, H), np.uint16)
    xp[src >= 0] = x[src[src >= 0]]
    out = host(mxa.combine(dev(xp), dev(dst), dev(np.ones((T, 1), np.float32)), T, 1))
    assert np.array_equal(out, x)


@pytest.mark.parametrize("T,H,E,topk,dup", [(300, 96, 6, 2, False), (128, 2048, 16, 8, False),
                                            (77, 544, 4, 3, True), (40, 160, 64, 9, False),
                                            (50, 96, 128, 64, False), (200, 416, 8, 4, True)])
def test_combine_bwd_quantize(T, H, E, topk, dup):
    g = np.random.default_rng(T + H + topk)
    ids, w, off, dst, src = routed(g, T, E, topk, dup)
    w[0, 0] = 0.0                                    # a zero weight: signed zeros
    w[1, :] = np.float32(1.0 / 3.0)                  # products that need fp32 rounding
    rows = src.size
    dout = workloads.normal_bf16(g, (T, H), 1.0, outlier_p=0.01)
    dout[2, :8] = mx.f64_to_bf16(np.array([1e-38, -1e-38, 3e-39, 1e-40, 0.0, -0.0, 1e30, -1e30]))
    dy, rq, rs, cq, cs = mxa.combine_bwd_quantize(dev(dout), dev(w), dev(dst), dev(src), topk, rows,
                                                  rowwise=True, colwise=True, want_bf16=True)
    torch.cuda.synchronize()
    dyb = host(dy)
    want = glue.combine_bwd(dout, dst, w, topk, rows)
    assert np.array_equal(dyb, want)
    check_mx(want, rq, rs, cq, cs)
    _, rq2, rs2, cq2, cs2 = mxa.combine_bwd_quantize(dev(dout), dev(w), dev(dst), dev(src), topk, rows,
                                                     rowwise=True, colwise=True, want_bf16=False)
    torch.cuda.synchronize()
    for u, v in ((rq, rq2), (rs, rs2), (cq, cq2), (cs, cs2)):
        assert torch.equal(u, v)


def test_combine_bwd_misaligned_metadata_same_bytes():
    """Top-8 pair lookup with dst_row and weights at 4-byte (not 16-byte)
    aligned addresses takes the scalar path; the bytes are the same."""
    g = np.random.default_rng(5)
    T, H, E, topk = 96, 544, 16, 8
    ids, w, off, dst, src = routed(g, T, E, topk)
    rows = src.size
    dout_np = workloads.normal_bf16(g, (T, H), 1.0, outlier_p=0.01)
    dout = dev(dout_np)
    a = mxa.combine_bwd_quantize(dout, dev(w), dev(dst), dev(src), topk, rows, rowwise=True, colwise=True,
                                 want_bf16=True)
    dst_m = torch.zeros(dst.size + 1, dtype=torch.int32, device="cuda:0")
    w_m = torch.zeros(w.size + 1, dtype=torch.float32, device="cuda:0")
    dst_m[1:] = dev(dst.ravel())
    w_m[1:] = dev(w.ravel())
    assert dst_m[1:].data_ptr() % 16 and w_m[1:].data_ptr() % 16
    b = mxa.combine_bwd_quantize(dout, w_m[1:], dst_m[1:], dev(src), topk, rows, rowwise=True, colwise=True,
                                 want_bf16=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    assert np.array_equal(host(a[0]), glue.combine_bwd(dout_np, dst, w, topk, rows))


def test_glue_empty_inputs():
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    a, rq, rs, cq, cs = mxa.swiglu_quantize(e, want_bf16=True)
    assert a.shape == (0, 32) and rq.shape == (0, 32)
    out = mxa.combine(torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda:0"),
                      torch.empty(0, dtype=torch.int32, device="cuda:0"), None, 0, 2)
    assert out.shape == (0, 64)
    torch.cuda.synchronize()


def test_combine_bwd_without_tokens_gives_zero_rows():
    src = torch.full((64,), -1, dtype=torch.int32, device="cuda:0")
    dout = torch.empty((0, 96), dtype=torch.bfloat16, device="cuda:0")
    dy, rq, rs, cq, cs = mxa.combine_bwd_quantize(dout, None, None, src, 2, 64, want_bf16=True)
    torch.cuda.synchronize()
    for t in (dy, rq, rs, cq, cs):
        assert not host(t).any()
