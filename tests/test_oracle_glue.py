"""Pins for the glue oracle (CPU only): SwiGLU and its backward, the weighted
unpermute-combine and its backward.  The pins come from outside the oracle's
own formulas: a library sigmoid, finite differences of the forward, the
closed-form minimum of SiLU (Lambert W), the adjoint identity between the
combine and its backward, the permute round trip, and a hand-derived case.
"""

import json
import os

import numpy as np
import scipy.special as sp

import workloads
from oracle import glue
from oracle import mxfp8 as mx
from oracle import routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(v):
    return mx.f64_to_bf16(np.asarray(v, dtype=np.float64))


# --------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------
def test_sigmoid_matches_library():
    x = np.linspace(-700, 700, 20001)
    np.testing.assert_allclose(glue.sigmoid(x), sp.expit(x), rtol=1e-14, atol=0)
    assert glue.sigmoid(np.array([-1e4]))[0] == 0.0
    assert glue.sigmoid(np.array([0.0]))[0] == 0.5


def test_silu_odd_part_identity():
    # silu(x) - silu(-x) = x  (sigmoid(x) + sigmoid(-x) = 1)
    x = np.random.default_rng(0).normal(0, 5, 10000)
    np.testing.assert_allclose(glue.silu(x) - glue.silu(-x), x, rtol=1e-13, atol=1e-13)


def test_silu_minimum_is_lambert_w():
    # d/dx silu = sigmoid(x) (1 + x (1 - sigmoid(x))) vanishes at x* = -1 - W(1/e),
    # where silu(x*) = -W(1/e).
    w = sp.lambertw(np.exp(-1.0)).real
    xs = -1.0 - w
    assert abs(glue.silu(xs) + w) < 1e-15
    F = 1
    h = np.array([[0, 0]], dtype=np.uint16)  # placeholder shape, values below
    g = np.array([[xs]])
    u = np.array([[1.0]])
    s = glue.sigmoid(g)
    assert abs((s * (1 + g * (1 - s)))[0, 0]) < 1e-15
    # the oracle's dg at the nearest bf16 to x* is tiny compared with its S
    h = np.concatenate([bf16(g), bf16(u)], axis=1)
    dh, S = glue.swiglu_bwd(h, bf16([[1.0]]), F)
    assert abs(dh[0, 0]) < 2e-3 * S[0, 0]


def test_swiglu_closed_forms_at_zero():
    h = np.concatenate([bf16(np.zeros((1, 4))), bf16([[1.0, -2.0, 3.5, 0.0]])], axis=1)
    a, _ = glue.swiglu(h, 4)
    assert np.all(a == 0)
    dh, _ = glue.swiglu_bwd(h, bf16([[2.0, 2.0, -1.0, 5.0]]), 4)
    # sigmoid(0) = 1/2, silu'(0) = 1/2: dg = dA u / 2, du = dA silu(0) = 0
    np.testing.assert_array_equal(dh[0, :4], [1.0, -2.0, -1.75, 0.0])
    np.testing.assert_array_equal(dh[0, 4:], 0.0)


def test_swiglu_bwd_is_the_derivative():
    """Central differences of the fp64 forward in g and in u."""
    g_ = np.random.default_rng(1)
    F, R = 64, 16
    h = workloads.normal_bf16(g_, (R, 2 * F), 2.0)
    da = workloads.normal_bf16(g_, (R, F))
    dh, S = glue.swiglu_bwd(h, da, F)
    g = mx.bf16_to_f64(h[:, :F])
    u = mx.bf16_to_f64(h[:, F:])
    d = mx.bf16_to_f64(da)
    eps = 1e-6 * np.maximum(1.0, np.abs(g))
    fd_g = d * (glue.silu(g + eps) * u - glue.silu(g - eps) * u) / (2 * eps)
    fd_u = d * glue.silu(g)   # A is linear in u: the difference quotient is exact
    fd_u2 = d * (glue.silu(g) * (u + 0.5) - glue.silu(g) * (u - 0.5))
    np.testing.assert_allclose(dh[:, :F], fd_g, rtol=0, atol=1e-7 * S[:, :F].max())
    assert np.all(np.abs(dh[:, :F] - fd_g) <= 1e-6 * S[:, :F] + 1e-12)
    np.testing.assert_allclose(dh[:, F:], fd_u, rtol=1e-15)
    np.testing.assert_allclose(dh[:, F:], fd_u2, rtol=1e-12, atol=1e-12)


def test_swiglu_large_magnitudes_are_finite():
    h = np.concatenate([bf16([[-1e30, 1e30, -100.0, 100.0]]), bf16([[1.0, 1.0, 1.0, 1.0]])], axis=1)
    a, _ = glue.swiglu(h, 4)
    assert np.all(np.isfinite(a))
    assert a[0, 0] == 0.0 and a[0, 1] == mx.bf16_to_f64(bf16([1e30]))[0]
    dh, S = glue.swiglu_bwd(h, bf16([[1.0, 1.0, 1.0, 1.0]]), 4)
    assert np.all(np.isfinite(dh)) and np.all(np.isfinite(S))


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------
def test_combine_golden():
    with open(os.path.join(GOLDEN, "combine_small.json")) as fh:
        gd = json.load(fh)
    rows = gd["rows"]
    y = np.zeros((rows, 2))
    y[:, 0] = np.arange(rows)
    y[:, 1] = 1.0
    out, S = glue.combine(bf16(y), gd["dst_row"], np.array(gd["weights"], np.float32), gd["topk"])
    np.testing.assert_array_equal(out, np.array(gd["out"]))
    dy = glue.combine_bwd(bf16(gd["dout"]), gd["dst_row"], np.array(gd["weights"], np.float32),
                          gd["topk"], rows)
    want = np.zeros((rows, 2), dtype=np.uint16)
    for r, v in gd["dy_rows"].items():
        want[int(r)] = [0x8000 if x == "-0" else int(bf16([x])[0]) for x in v]
    np.testing.assert_array_equal(dy, want)
    assert dy[66, 1] == 0x8000 and dy[66, 0] == 0x0000


def test_combine_is_inverse_of_permute_for_top1():
    g = np.random.default_rng(2)
    T, H, E = 200, 96, 5
    ids = g.integers(0, E, (T, 1))
    _, off, dst, src = routing.route(ids, E)
    x = workloads.normal_bf16(g, (T, H))
    xp = np.zeros((src.size, H), dtype=np.uint16)
    xp[src >= 0] = x[src[src >= 0]]
    out, _ = glue.combine(xp, dst, np.ones((T, 1), np.float32), 1)
    np.testing.assert_array_equal(out, mx.bf16_to_f64(x))
    out2, _ = glue.combine(xp, dst, None, 1)
    np.testing.assert_array_equal(out2, out)


def test_combine_bwd_is_the_adjoint():
    """<combine(Y), dOut> = <Y, combine_bwd(dOut)> for any Y, dOut."""
    g = np.random.default_rng(3)
    T, H, E, k = 64, 32, 6, 3
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)])
    _, off, dst, src = routing.route(ids, E)
    rows = src.size
    w = g.random((T, k)).astype(np.float32)
    y = workloads.normal_bf16(g, (rows, H))
    dout = g.normal(size=(T, H))
    out, _ = glue.combine(y, dst, w, k)
    dy = glue.combine_bwd_exact(dout, dst, w, k, rows)
    lhs = np.sum(out * dout)
    rhs = np.sum(mx.bf16_to_f64(y) * dy)
    assert abs(lhs - rhs) <= 1e-12 * np.sum(np.abs(out) * np.abs(dout))
    # unmapped (pad) rows of the backward are zero
    assert np.all(dy[src < 0] == 0)


def test_combine_convex_weights_of_equal_rows():
    g = np.random.default_rng(4)
    T, H, k = 40, 64, 4
    dst = g.permutation(T * k + 7)[:T * k]
    v = workloads.normal_bf16(g, (T, H))
    y = np.zeros((T * k + 7, H), dtype=np.uint16)
    for i in range(T * k):
        y[dst[i]] = v[i // k]
    w = g.random((T, k))
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    out, S = glue.combine(y, dst, w, k)
    np.testing.assert_allclose(out, mx.bf16_to_f64(v) * w.astype(np.float64).sum(1, keepdims=True), rtol=1e-15)
    np.testing.assert_allclose(S, np.abs(out), rtol=1e-15)


def test_combine_bwd_rounds_the_fp32_product():
    # w = 1/3 in fp32 is not a power of two: the fp32 product of w and a bf16
    # value needs rounding, and the bf16 result is the RNE of that fp32 value.
    w = np.array([[np.float32(1.0 / 3.0)]], np.float32)
    d = bf16([[3.0, 1.5, -7.0, 1e-38]])
    dy = glue.combine_bwd(d, [0], w, 1, 1)
    p = (np.float32(1.0 / 3.0) * mx.bf16_to_f64(d).astype(np.float32)).astype(np.float64)
    np.testing.assert_array_equal(dy[0], bf16(p)[0])
    # exact powers of two: the bf16 result is the exact product
    dy2 = glue.combine_bwd(d, [0], np.array([[0.25]], np.float32), 1, 1)
    np.testing.assert_array_equal(dy2[0], bf16(mx.bf16_to_f64(d)[0] * 0.25))


def test_glue_rule_accepts_rne_and_rejects_two_ulps():
    from oracle import tolerance
    g = np.random.default_rng(5)
    v = g.normal(size=1000)
    rne = bf16(v)
    assert tolerance.check_bf16_elementwise(rne, v, np.abs(v))["ok"]
    off2 = (rne.astype(np.int64) + 2).astype(np.uint16)     # two bf16 ulps away (same binade mostly)
    assert not tolerance.check_bf16_elementwise(off2, v, np.abs(v))["ok"]
