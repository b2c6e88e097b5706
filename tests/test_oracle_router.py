"""Pins for the router oracle (CPU only): the top-k rule by an independent
rank characterisation, the weights against SciPy's softmax, shift
invariance and ties, and the backward against finite differences of the
layer output's inner product with dOut."""

import numpy as np
import scipy.special as sp

import workloads
from oracle import glue
from oracle import mxfp8 as mx
from oracle import router


def test_topk_rank_characterisation():
    g = np.random.default_rng(0)
    lg = g.standard_normal((300, 12)).astype(np.float32)
    lg[:20, 3] = lg[:20, 7]              # exact ties between experts 3 and 7
    lg[20:30] = 0.5                      # all equal
    ids, w = router.route_topk(lg, 4)
    for t in range(lg.shape[0]):
        for j, e in enumerate(ids[t]):
            better = np.sum((lg[t] > lg[t, e]) | ((lg[t] == lg[t, e]) & (np.arange(12) < e)))
            assert better == j
    assert np.array_equal(ids[20:30], np.tile(np.arange(4), (10, 1)))
    np.testing.assert_allclose(w[20:30], 0.25, rtol=1e-15)


def test_weights_are_softmax_of_chosen():
    g = np.random.default_rng(1)
    lg = (np.round(g.standard_normal((200, 64)) * 3 * 64) / 64).astype(np.float32)   # 6 fraction bits: +16 is exact
    ids, w = router.route_topk(lg, 8)
    ref = sp.softmax(np.take_along_axis(lg.astype(np.float64), ids, 1), axis=1)
    np.testing.assert_allclose(w, ref, rtol=1e-14)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    ids2, w2 = router.route_topk(lg + np.float32(16.0), 8)   # an exact shift of every logit
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w2, w, rtol=1e-13)
    ids3, w3 = router.route_topk(lg + np.float32(1000.0), 8)  # large logits: no overflow
    assert np.array_equal(ids, ids3) and np.all(np.isfinite(w3))
    np.testing.assert_allclose(w3, w, rtol=1e-13)
    idsk, wk = router.route_topk(lg[:5], 64)                 # k = E: the full softmax
    np.testing.assert_allclose(np.take_along_axis(wk, np.argsort(idsk, 1), 1),
                               sp.softmax(lg[:5].astype(np.float64), axis=1), rtol=1e-13)


def layer_out(lg64, ids, y, dst, topk):
    """Combine output with the softmax weights of fixed ids, as a function of fp64 logits."""
    z = np.take_along_axis(lg64, ids, 1)
    w = sp.softmax(z, axis=1)
    T = ids.shape[0]
    rows = np.asarray(dst).reshape(T, topk)
    return np.einsum("tj,tjh->th", w, y[rows])


def test_router_bwd_matches_finite_differences():
    g = np.random.default_rng(2)
    T, E, k, H = 24, 10, 3, 32
    lg = g.standard_normal((T, E)).astype(np.float32)
    ids, w = router.route_topk(lg, k)
    rows = T * k + 5
    dst = g.permutation(rows)[:T * k]
    yb = workloads.normal_bf16(g, (rows, H))
    db = workloads.normal_bf16(g, (T, H))
    y, d = mx.bf16_to_f64(yb), mx.bf16_to_f64(db)
    dw, sdw, dl, sl = router.router_bwd(db, yb, dst, ids, w.astype(np.float32), E)
    # dw: the combine is linear in w
    for t, j in [(0, 0), (5, 2), (23, 1)]:
        np.testing.assert_allclose(dw[t, j], d[t] @ y[dst[t * k + j]], rtol=1e-13)
    # dlogits: central differences of <dOut, out(logits)> (ids held fixed)
    lg64 = lg.astype(np.float64)
    # with the fp64 softmax weights the logit gradient is the exact derivative
    dw64, _, dl64, _ = router.router_bwd(db, yb, dst, ids, w, E)
    eps = 1e-6
    for t in range(0, T, 5):
        for e in range(E):
            p = lg64.copy(); p[t, e] += eps
            m = lg64.copy(); m[t, e] -= eps
            fd = (np.sum(d * layer_out(p, ids, y, dst, k)) - np.sum(d * layer_out(m, ids, y, dst, k))) / (2 * eps)
            assert abs(fd - dl64[t, e]) <= 1e-6 * (sl[t].max() + 1e-12)
    # softmax gradients sum to zero over the experts of a token; unchosen experts get 0
    np.testing.assert_allclose(dl64.sum(1), 0.0, atol=1e-12 * sl.max())
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids, True, 1)
    assert np.all(dl[~mask] == 0)


def test_router_bwd_consistent_with_glue_combine():
    g = np.random.default_rng(3)
    T, E, k, H = 16, 8, 2, 64
    lg = g.standard_normal((T, E)).astype(np.float32)
    ids, w = router.route_topk(lg, k)
    rows = T * k
    dst = g.permutation(rows)
    yb = workloads.normal_bf16(g, (rows, H))
    db = workloads.normal_bf16(g, (T, H))
    dw, _, _, _ = router.router_bwd(db, yb, dst, ids, w.astype(np.float32), E)
    # <dOut, combine(Y, w)> = sum_tj w_tj dw_tj  (the weight gradient is the combine's coefficient)
    out, _ = glue.combine(yb, dst, w.astype(np.float32), k)
    lhs = np.sum(mx.bf16_to_f64(db) * out)
    rhs = np.sum(w.astype(np.float32).astype(np.float64) * dw)
    assert abs(lhs - rhs) <= 1e-12 * np.sum(np.abs(mx.bf16_to_f64(db)) @ np.abs(mx.bf16_to_f64(yb)).T)
