"""Pins for the BF16-baseline oracle (CPU only): brute-force triple loops
that decode bf16 with torch's own bfloat16 and sum with math.fsum, closed
forms, the empty-expert case, gather/transpose index brute force, and the
agreement of the BF16 and MXFP8 oracles on operands both represent exactly
(the MX values of E4M3 codes with in-range scales are bf16 values)."""

import math

import numpy as np
import torch

from oracle import bf16 as ob
from oracle import gemm as og
from oracle import mxfp8 as mx


def t_bf16(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def rand_bf16(g, shape, std=1.0):
    v = g.standard_normal(shape) * std
    return mx.f64_to_bf16(v)


def test_fwd_brute_force_and_empty_group():
    g = np.random.default_rng(11)
    M, N, K, E = 80, 6, 64, 3
    a = rand_bf16(g, (M, K))
    b = rand_bf16(g, (E, N, K), 0.02)
    off = np.array([0, 32, 32, 80])                      # expert 1 empty
    C, S = ob.grouped_gemm_rows(a, b, off)
    A, B = t_bf16(a), t_bf16(b)
    for m in range(M):
        e = 0 if m < 32 else 2
        for n in range(N):
            terms = [A[m, k] * B[e, n, k] for k in range(K)]
            assert math.isclose(C[m, n], math.fsum(terms), rel_tol=1e-13, abs_tol=1e-300)
            assert math.isclose(S[m, n], math.fsum(abs(t) for t in terms), rel_tol=1e-13)


def test_rows_outside_groups_are_zero():
    g = np.random.default_rng(12)
    a = rand_bf16(g, (96, 32))
    b = rand_bf16(g, (2, 4, 32))
    C, S = ob.grouped_gemm_rows(a, b, np.array([32, 40, 64]))
    assert not C[:32].any() and not C[64:].any() and not S[64:].any()
    assert C[32:64].any()


def test_wgrad_brute_force_and_empty_group():
    g = np.random.default_rng(13)
    N, K, Mc = 5, 7, 128
    dyt = rand_bf16(g, (N, Mc))
    xt = rand_bf16(g, (K, Mc))
    off = np.array([0, 64, 64, 128])
    C, S = ob.grouped_gemm_wgrad(dyt, xt, off)
    assert C.shape == (3, N, K) and np.all(C[1] == 0) and np.all(S[1] == 0)
    DY, X = t_bf16(dyt), t_bf16(xt)
    for e, (lo, hi) in enumerate([(0, 64), (64, 64), (64, 128)]):
        for n in range(N):
            for k in range(K):
                terms = [DY[n, r] * X[k, r] for r in range(lo, hi)]
                assert math.isclose(C[e, n, k], math.fsum(terms), rel_tol=1e-13, abs_tol=1e-300)


def test_ones_give_column_sums():
    # A of 1.0 (0x3F80): every output row is the row sum of B_e over k
    g = np.random.default_rng(14)
    a = np.full((64, 96), 0x3F80, np.uint16)
    b = rand_bf16(g, (2, 8, 96))
    C, _ = ob.grouped_gemm_rows(a, b, np.array([0, 32, 64]))
    B = t_bf16(b)
    np.testing.assert_allclose(C[:32], np.broadcast_to(B[0].sum(1), (32, 8)), rtol=1e-14)
    np.testing.assert_allclose(C[32:], np.broadcast_to(B[1].sum(1), (32, 8)), rtol=1e-14)


def test_dgrad_is_fwd_on_transposed_weight():
    # dX = dY . W_e, with W_e entering as its transpose [K, N]
    g = np.random.default_rng(15)
    M, N, K = 64, 32, 96
    dy = rand_bf16(g, (M, N))
    w = rand_bf16(g, (1, N, K), 0.02)
    C, _ = ob.grouped_gemm_rows(dy, ob.transpose(w[0])[None], np.array([0, M]))
    DY, W = t_bf16(dy), t_bf16(w[0])
    for m in range(0, M, 5):
        for k in range(0, K, 7):
            assert math.isclose(C[m, k], math.fsum(DY[m, n] * W[n, k] for n in range(N)), rel_tol=1e-13,
                                abs_tol=1e-300)


def test_agrees_with_mx_oracle_on_mx_values():
    # E4M3 codes with scales 2^-10..2^4 decode to bf16 values exactly (3
    # mantissa bits, exponents well inside bf16's range); the BF16 product of
    # those values is the MX product.
    g = np.random.default_rng(16)
    M, N, K = 64, 8, 128
    aq = g.integers(0, 0x7F, (M, K)).astype(np.uint8) | (g.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    bq = g.integers(0, 0x7F, (2, N, K)).astype(np.uint8)
    as_ = g.integers(117, 131, (M, K // 32)).astype(np.uint8)
    bs = g.integers(117, 131, (2, N, K // 32)).astype(np.uint8)
    av, bv = mx.mx_values(aq, as_), mx.mx_values(bq, bs)
    a16, b16 = mx.f64_to_bf16(av), mx.f64_to_bf16(bv)
    assert np.array_equal(mx.bf16_to_f64(a16), av) and np.array_equal(mx.bf16_to_f64(b16), bv)
    off = np.array([0, 32, 64])
    C16, S16 = ob.grouped_gemm_rows(a16, b16, off)
    Cmx, Smx = og.grouped_gemm_fwd(aq, as_, bq, bs, off)
    np.testing.assert_allclose(C16, Cmx, rtol=0, atol=1e-12 * np.abs(Smx).max())
    np.testing.assert_allclose(S16, Smx, rtol=1e-14)


def test_gather_and_transpose_by_index():
    g = np.random.default_rng(17)
    x = g.integers(0, 1 << 16, (10, 32)).astype(np.uint16)
    idx = np.array([3, -1, 9, 10, 0, 0, 1000, 2])
    out = ob.gather(x, idx, 8)
    for r, s in enumerate(idx):
        if 0 <= s < 10:
            assert np.array_equal(out[r], x[s])
        else:
            assert not out[r].any()
    pad = ob.gather(x, None, 16)
    assert np.array_equal(pad[:10], x) and not pad[10:].any()
    t = ob.transpose(pad)
    assert t.shape == (32, 16)
    for r in range(16):
        for c in range(32):
            assert t[c, r] == pad[r, c]
