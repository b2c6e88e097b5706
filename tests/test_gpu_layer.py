"""GPU parity of the whole SwiGLU expert FFN layer at full size (32768 tokens,
top-8 of 64 experts, hidden 7168, expert ffn 2048), run exactly as the
benchmark runs it (``moe.layer_step`` on ``workloads.layer_inputs``), checked
stage by stage on sampled outputs that the oracle computes one by one from
the bytes each stage consumed:

* routing in full and every sampled MX byte bit-exact;
* GEMM elements under the pass rule of oracle/tolerance.py (with the
  hardware term), from the kernel's own MX operand bytes;
* the glue's bf16 values under the element-wise glue rule, and their MX
  bytes bit-exact against the oracle's quantize of those values.
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from mxfp8_block_scaled_07_amd import moe
from oracle import glue
from oracle import mxfp8 as mx
from oracle import router, routing, tolerance

from gpu_util import host

pytestmark = pytest.mark.gpu


def ix(a):
    return torch.from_numpy(np.asarray(a, np.int64)).cuda()


def rows(t, r):
    """Rows r of a device tensor, on the host (bf16 as uint16 bits)."""
    return host(t[ix(r)])


def cols(t, c):
    return host(t[:, ix(c)])


def srow_sel(sp, C, r):
    """Row-major scale bytes [len(r), C/32] of rows r of a panel-layout scale tensor."""
    a = host(sp[:, ix(r), :])
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(len(r), -1)[:, :C // 32])


@pytest.fixture(scope="module")
def layer():
    inp = workloads.layer_inputs("cuda:0")
    T, H, F, E, k = inp["T"], inp["H"], inp["F"], inp["E"], inp["topk"]
    b = moe.LayerBuffers(T, H, F, E, k)
    moe.layer_step(b, inp["x"], inp["w1"], inp["w2"], inp["logits"], inp["dout"])
    torch.cuda.synchronize()
    ids, w = router.route_topk(host(inp["logits"]), k)
    assert np.array_equal(host(b.ids), ids)
    assert np.all(np.abs(host(b.weights) - w) <= 2.0 ** -20 * w)
    inp["weights"] = b.weights
    _, off, dst, src = routing.route(ids, E, b.cap)
    return inp, b, off, dst, src


def grade(name, got, aq, as_, bq, bs):
    """got: bf16 bits of sampled GEMM elements; (aq, as_), (bq, bs): the MX
    operand rows (codes [P, L], row-major scales [P, L/32]) of each element."""
    A, B = mx.mx_values(aq, as_), mx.mx_values(bq, bs)
    P = A * B
    C, S = P.sum(-1), np.abs(P).sum(-1)
    ea, eb = tolerance.nominal_exponents(aq, as_), tolerance.nominal_exponents(bq, bs)
    res = tolerance.check(got, C, S, h_fn=lambda i: tolerance.hardware_term(ea[i], eb[i]), out_bf16=True)
    print(name, res)
    assert res["ok"], (name, res)


def test_routing_and_quantized_inputs(layer):
    inp, b, off, dst, src = layer
    T, H, F, E = inp["T"], inp["H"], inp["F"], inp["E"]
    assert np.array_equal(host(b.off), off) and np.array_equal(host(b.dst), dst)
    assert np.array_equal(host(b.src), src)
    g = np.random.default_rng(51)
    # X rowwise, its permuted copy
    r = np.sort(g.choice(T, 64, replace=False))
    xr = rows(inp["x"], r)
    oq, os_ = mx.quantize_rowwise(xr)
    assert np.array_equal(rows(b.xq, r), oq) and np.array_equal(srow_sel(b.xs, H, r), os_)
    pr = np.sort(g.choice(np.nonzero(src >= 0)[0], 64, replace=False))
    oq, os_ = mx.quantize_rowwise(rows(inp["x"], src[pr]))
    assert np.array_equal(rows(b.xpq, pr), oq) and np.array_equal(srow_sel(b.xps, H, pr), os_)
    pad = np.nonzero(src < 0)[0][:16]
    assert not rows(b.xpq, pad).any()
    # W1 and W2, rowwise and columnwise, two experts
    for e in (0, int(g.integers(1, E))):
        for w, q, s, tq, ts, N, K in ((inp["w1"], b.w1q, b.w1s, b.w1tq, b.w1ts, 2 * F, H),
                                      (inp["w2"], b.w2q, b.w2s, b.w2tq, b.w2ts, H, F)):
            we = w[e]
            wr = np.sort(g.choice(N, 8, replace=False))
            oq, os_ = mx.quantize_rowwise(rows(we, wr))
            assert np.array_equal(rows(q[e], wr), oq) and np.array_equal(srow_sel(s, K, e * N + wr), os_)
            wc = np.sort(g.choice(K, 8, replace=False))
            cq, cs = mx.quantize_rowwise(np.ascontiguousarray(cols(we, wc).T))
            assert np.array_equal(rows(tq[e], wc), cq) and np.array_equal(srow_sel(ts, N, e * K + wc), cs)
    # X columnwise in permuted order (gather)
    xc = np.sort(g.choice(H, 6, replace=False))
    cq, cs = mx.quantize_colwise(cols(inp["x"], xc), rows_out=b.cap, gather=src)
    assert np.array_equal(rows(b.xtq, xc), cq) and np.array_equal(srow_sel(b.xts, b.cap, xc), cs)


def row_gemm_samples(g, b, off, src, n_out, nsamp=192):
    real = np.nonzero(src >= 0)[0]
    m = g.choice(real, nsamp)
    n = g.integers(0, n_out, nsamp)
    grp = np.searchsorted(off, m, side="right") - 1
    return m, n, grp


def test_gate_up_gemm_and_swiglu(layer):
    inp, b, off, dst, src = layer
    H, F = inp["H"], inp["F"]
    g = np.random.default_rng(52)
    m, n, grp = row_gemm_samples(g, b, off, src, 2 * F)
    got = host(b.h[ix(m), ix(n)])
    grade("gemm1_fwd", got, rows(b.xpq, m), srow_sel(b.xps, H, m), host(b.w1q[ix(grp), ix(n)]),
          srow_sel(b.w1s, H, grp * 2 * F + n))
    # SwiGLU on the GEMM's own H: the same kernel with the bf16 A written too
    a, aq, as_, atq, ats = mxa.swiglu_quantize(b.h, want_bf16=True)
    torch.cuda.synchronize()
    for u, v in ((aq, b.aq), (as_, b.as_), (atq, b.atq), (ats, b.ats)):
        assert torch.equal(u, v)
    r = np.sort(g.choice(b.cap, 96, replace=False))
    ab = rows(a, r)
    ex, S = glue.swiglu(rows(b.h, r), F)
    res = tolerance.check_bf16_elementwise(ab, ex, S)
    print("swiglu", res)
    assert res["ok"], res
    oq, os_ = mx.quantize_rowwise(ab)
    assert np.array_equal(rows(b.aq, r), oq) and np.array_equal(srow_sel(b.as_, F, r), os_)
    c = np.sort(g.choice(F, 6, replace=False))
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(cols(a, c).T))
    assert np.array_equal(rows(b.atq, c), cq) and np.array_equal(srow_sel(b.ats, b.cap, c), cs)


def test_down_gemm_and_combine(layer):
    inp, b, off, dst, src = layer
    H, F, k = inp["H"], inp["F"], inp["topk"]
    g = np.random.default_rng(53)
    m, n, grp = row_gemm_samples(g, b, off, src, H)
    got = host(b.y[ix(m), ix(n)])
    grade("gemm2_fwd", got, rows(b.aq, m), srow_sel(b.as_, F, m), host(b.w2q[ix(grp), ix(n)]),
          srow_sel(b.w2s, F, grp * H + n))
    ts = np.sort(g.choice(inp["T"], 48, replace=False))
    pairs = (ts[:, None] * k + np.arange(k)).ravel()
    w = host(inp["weights"])[ts]
    ysub = rows(b.y, dst[pairs])
    ex, S = glue.combine(ysub, np.arange(pairs.size), w, k)
    res = tolerance.check_bf16_elementwise(rows(b.out, ts), ex, S)
    print("combine", res)
    assert res["ok"], res


def test_combine_bwd_and_down_backward(layer):
    inp, b, off, dst, src = layer
    T, H, F, k = inp["T"], inp["H"], inp["F"], inp["topk"]
    g = np.random.default_rng(54)
    w = host(inp["weights"])
    # dY = combine backward: sampled columns over every row (rowwise and columnwise MX)
    c = np.sort(g.choice(H, 4, replace=False))
    dyc = glue.combine_bwd(cols(inp["dout"], c), dst, w, k, b.cap)
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(dyc.T))
    assert np.array_equal(rows(b.dytq, c), cq) and np.array_equal(srow_sel(b.dyts, b.cap, c), cs)
    r = np.sort(g.choice(b.cap, 48, replace=False))
    sel = np.nonzero(np.isin(dst, r))[0]
    local = np.searchsorted(r, dst[sel])
    tok = sel // k
    dyr = np.zeros((r.size, H), np.uint16)
    sub = glue.combine_bwd(rows(inp["dout"], tok), np.arange(sel.size), w.ravel()[sel], 1, sel.size)
    dyr[local] = sub
    oq, os_ = mx.quantize_rowwise(dyr)
    assert np.array_equal(rows(b.dyq, r), oq) and np.array_equal(srow_sel(b.dys, H, r), os_)
    # router backward: sampled tokens, from the kernel's own Y rows and weights
    ts = np.sort(g.choice(T, 32, replace=False))
    pairs = (ts[:, None] * k + np.arange(k)).ravel()
    edw, sdw, edl, sdl = glue_router_bwd(inp, b, ts, pairs, dst, k)
    rel = (H / 64 + 8) * 2.0 ** -24
    gdw, gdl = host(b.dweights)[ts], host(b.dlogits)[ts]
    assert np.all(np.abs(gdw - edw) <= rel * sdw + 2.0 ** -126), "router dw"
    assert np.all(np.abs(gdl - edl) <= rel * sdl + 2.0 ** -126), "router dlogits"
    # dA = dY W2 (dgrad), from the kernel's own dY rows and W2^T columnwise bytes
    m, f, grp = row_gemm_samples(g, b, off, src, F)
    got = host(b.da[ix(m), ix(f)])
    grade("gemm2_dgrad", got, rows(b.dyq, m), srow_sel(b.dys, H, m), host(b.w2tq[ix(grp), ix(f)]),
          srow_sel(b.w2ts, H, grp * F + f))
    # dW2[e] = dY_e^T A_e (wgrad over the group's rows)
    wgrad_samples(g, "gemm2_wgrad", b.dw2, off, b.dytq, b.dyts, b.atq, b.ats, H, F, b.cap)


def glue_router_bwd(inp, b, ts, pairs, dst, k):
    """The oracle's router backward for tokens ts, on the kernel's Y rows and weights."""
    ysub = rows(b.y, dst[pairs])
    return router.router_bwd(rows(inp["dout"], ts), ysub, np.arange(pairs.size), host(b.ids)[ts],
                             host(b.weights)[ts], inp["E"])


def wgrad_samples(g, name, dw, off, aq_t, as_t, bq_t, bs_t, N, K, cap, nsamp=96):
    E = off.size - 1
    sizes = np.diff(off)
    es = g.choice(np.nonzero(sizes > 0)[0], nsamp)
    n = g.integers(0, N, nsamp)
    kk = g.integers(0, K, nsamp)
    got = host(dw[ix(es), ix(n), ix(kk)])
    L = int(sizes.max())
    A_all, As_all = rows(aq_t, n), srow_sel(as_t, cap, n)
    B_all, Bs_all = rows(bq_t, kk), srow_sel(bs_t, cap, kk)
    aq = np.zeros((nsamp, L), np.uint8)
    bq = np.zeros((nsamp, L), np.uint8)
    as_ = np.zeros((nsamp, L // 32), np.uint8)
    bs = np.zeros((nsamp, L // 32), np.uint8)
    for i, e in enumerate(es):
        lo, hi = int(off[e]), int(off[e + 1])
        aq[i, :hi - lo] = A_all[i, lo:hi]
        bq[i, :hi - lo] = B_all[i, lo:hi]
        as_[i, :(hi - lo) // 32] = As_all[i, lo // 32:hi // 32]
        bs[i, :(hi - lo) // 32] = Bs_all[i, lo // 32:hi // 32]
    grade(name, got, aq, as_, bq, bs)
    for e in np.nonzero(sizes == 0)[0]:
        assert torch.count_nonzero(dw[int(e)]) == 0


def test_swiglu_backward_and_gate_up_backward(layer):
    inp, b, off, dst, src = layer
    T, H, F, k = inp["T"], inp["H"], inp["F"], inp["topk"]
    g = np.random.default_rng(55)
    dh, dq, ds, dtq, dts = mxa.swiglu_bwd_quantize(b.h, b.da, want_bf16=True)
    torch.cuda.synchronize()
    for u, v in ((dq, b.dhq), (ds, b.dhs), (dtq, b.dhtq), (dts, b.dhts)):
        assert torch.equal(u, v)
    r = np.sort(g.choice(b.cap, 96, replace=False))
    dhb = rows(dh, r)
    ex, S = glue.swiglu_bwd(rows(b.h, r), rows(b.da, r), F)
    res = tolerance.check_bf16_elementwise(dhb, ex, S)
    print("swiglu_bwd", res)
    assert res["ok"], res
    oq, os_ = mx.quantize_rowwise(dhb)
    assert np.array_equal(rows(b.dhq, r), oq) and np.array_equal(srow_sel(b.dhs, 2 * F, r), os_)
    c = np.sort(g.choice(2 * F, 6, replace=False))
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(cols(dh, c).T))
    assert np.array_equal(rows(b.dhtq, c), cq) and np.array_equal(srow_sel(b.dhts, b.cap, c), cs)
    # dX_perm = dH W1 (dgrad over 2F)
    m, hh, grp = row_gemm_samples(g, b, off, src, H)
    got = host(b.dxp[ix(m), ix(hh)])
    grade("gemm1_dgrad", got, rows(b.dhq, m), srow_sel(b.dhs, 2 * F, m), host(b.w1tq[ix(grp), ix(hh)]),
          srow_sel(b.w1ts, 2 * F, grp * H + hh))
    # dW1[e] = dH_e^T X_e
    wgrad_samples(g, "gemm1_wgrad", b.dw1, off, b.dhtq, b.dhts, b.xtq, b.xts, 2 * F, H, b.cap)
    # dX = unweighted combine of dX_perm
    ts = np.sort(g.choice(T, 48, replace=False))
    pairs = (ts[:, None] * k + np.arange(k)).ravel()
    ex, S = glue.combine(rows(b.dxp, dst[pairs]), np.arange(pairs.size), None, k)
    res = tolerance.check_bf16_elementwise(rows(b.dx, ts), ex, S)
    print("unpermute_dx", res)
    assert res["ok"], res


def test_fused_layer_matches_full_path():
    """The layer step with the quantize fused into the permute writes the same
    bytes as the full path (top-8 of 64 experts, reduced sizes): routing,
    the permuted rowwise MX and columnwise MX of X, the layer output and the
    gradients of X, W1, W2 and the router logits."""
    inp = workloads.layer_inputs("cuda:0", T=2048, H=512, F=256, E=64, topk=8)
    T, H, F, E, k = inp["T"], inp["H"], inp["F"], inp["E"], inp["topk"]
    a = moe.LayerBuffers(T, H, F, E, k)
    f = moe.LayerBuffers(T, H, F, E, k)
    args = (inp["x"], inp["w1"], inp["w2"], inp["logits"], inp["dout"])
    moe.layer_step(a, *args)
    moe.fused_layer_step(f, *args)
    torch.cuda.synchronize()
    hi = int(a.off[-1])
    for name in ("ids", "weights", "off", "dst", "src", "xtq", "xts", "out", "dx", "dw1", "dw2", "dlogits"):
        ta, tf = getattr(a, name), getattr(f, name)
        if ta.dtype in (torch.bfloat16, torch.float32):
            ta, tf = ta.view(torch.int16 if ta.dtype == torch.bfloat16 else torch.int32), \
                tf.view(torch.int16 if tf.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(ta, tf), name
    assert torch.equal(a.xpq[:hi], f.xpq[:hi])
