"""Pins for the routing / permute oracle (CPU only): a hand-derived case,
brute force on tiny random tables and the permutation invariants.  The
token shuffle stays in MXFP8 (pytorch/ao PR #3203, "Next steps"); codes and
scales travel together (TransformerEngine issue #556, first maintainer reply).
"""

import json
import os

import numpy as np

from oracle import mxfp8 as mx
from oracle import routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_route_golden():
    with open(os.path.join(GOLDEN, "route_small.json")) as fh:
        g = json.load(fh)
    counts, offsets, dst, src = routing.route(np.array(g["expert_ids"]), g["num_experts"])
    assert list(counts) == g["counts"] and list(offsets) == g["offsets"]
    assert list(dst) == g["dst_row"] and src.size == g["capacity_rows"]
    want = np.full(src.size, -1)
    for r, t in g["src_row_nonneg"].items():
        want[int(r)] = t
    assert np.array_equal(src, want)


def brute_dst(ids, E):
    """For every pair, count the rows before it: all padded groups of lower
    experts plus earlier pairs of the same expert (direct definition)."""
    flat = ids.reshape(-1)
    out = []
    for i, e in enumerate(flat):
        base = 0
        for e2 in range(e):
            n = sum(1 for x in flat if x == e2)
            base += -(-n // 32) * 32
        out.append(base + sum(1 for x in flat[:i] if x == e))
    return np.array(out)


def test_route_brute_force_tiny():
    g = np.random.default_rng(4)
    for trial in range(30):
        T, k, E = int(g.integers(1, 40)), int(g.integers(1, 4)), int(g.integers(1, 6))
        ids = g.integers(0, E, (T, k))
        counts, offsets, dst, src = routing.route(ids, E)
        assert np.array_equal(dst, brute_dst(ids, E))
        assert counts.sum() == T * k and np.all(offsets % 32 == 0)


def test_route_invariants_and_permute():
    g = np.random.default_rng(8)
    T, k, E, K = 300, 3, 7, 64
    ids = g.integers(0, E, (T, k))
    ids[:, 0] = np.where(ids[:, 0] == 5, 6, ids[:, 0])
    ids[:, 1:] = np.where(ids[:, 1:] == 5, 4, ids[:, 1:])          # expert 5 empty
    counts, offsets, dst, src = routing.route(ids, E)
    assert counts[5] == 0 and offsets[5] == offsets[6]
    assert len(set(dst.tolist())) == T * k                         # injective
    assert np.array_equal(src[dst], np.arange(T * k) // k)         # inverse
    assert np.all(np.bincount(src[src >= 0], minlength=T) == k)    # each token k times
    for e in range(E):                                             # rows inside their group, stable
        rows = dst[ids.reshape(-1) == e]
        assert np.all((rows >= offsets[e]) & (rows < offsets[e] + counts[e]))
        assert np.all(np.diff(rows) == 1)
    x = (g.standard_normal((T, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s = mx.quantize_rowwise(x)
    qp, sp = routing.permute(q, s, src)
    # permute(quantize(X)) == quantize(permute(X)): rowwise quantization commutes with row moves
    xp = mx.gather_rows(x, src, src.size)
    q2, s2 = mx.quantize_rowwise(xp)
    assert np.array_equal(qp, q2) and np.array_equal(sp, s2)
    pad = src < 0
    assert np.all(qp[pad] == 0) and np.all(sp[pad] == 0)
