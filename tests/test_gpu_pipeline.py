"""GPU parity of the whole expert path at the large workload's full size
(8192 tokens x 5120 hidden, top-2 of 16 experts with one empty expert, ffn
8192, 0.1% outliers x1000), run exactly as the benchmark runs it
(``moe.expert_step``), checked on sampled outputs the oracle computes one by
one from the bf16 inputs: quantized bytes bit-exact, routing bit-exact in
full, GEMM elements under the tolerance rule of oracle/tolerance.py."""

import numpy as np
import pytest
import torch

import workloads
from mxfp8_block_scaled_07_amd import MX_OUT_BF16, MX_OUT_F32, moe
from oracle import mxfp8 as mx
from oracle import routing, tolerance

from gpu_util import dev, host, srows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    c = workloads.config(3)
    T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
    x, w, ids = dev(c["x"]), dev(c["w"]), dev(c["expert_ids"])
    counts, off, dst, src = routing.route(c["expert_ids"], E, c["capacity"])
    dy_np = c["dy_full"].copy()
    dy_np[src < 0] = 0                       # pad rows of the padded permuted layout
    return c, x, w, ids, dev(dy_np), dy_np, (counts, off, dst, src)


def bf16_f64(b):
    return mx.bf16_to_f64(b)


@pytest.mark.parametrize("out_dtype", [MX_OUT_BF16, MX_OUT_F32])
def test_expert_step_full_size(case, out_dtype):
    c, x, w, ids, dy, dy_np, (counts, off, dst, src) = case
    T, K, N, E, topk, cap = c["T"], c["K"], c["N"], c["E"], c["topk"], c["capacity"]
    b = moe.ExpertBuffers(T, K, N, E, topk, out_dtype=out_dtype)
    assert b.cap == cap
    moe.expert_step(b, x, w, dy, ids)
    torch.cuda.synchronize()
    g = np.random.default_rng(2024 + out_dtype)

    # routing: full, bit-exact
    assert np.array_equal(host(b.off), off) and np.array_equal(host(b.dst), dst)
    assert np.array_equal(host(b.src), src)
    empty = [e for e in range(E) if counts[e] == 0]
    assert empty, "the workload forces one empty expert"

    # X rowwise and its permuted copy (sampled rows)
    rows = np.sort(g.choice(T, 64, replace=False))
    oq, os_ = mx.quantize_rowwise(c["x"][rows])
    assert np.array_equal(host(b.xq)[rows], oq) and np.array_equal(srows(b.xs, K)[rows], os_)
    prow = np.sort(g.choice(cap, 128, replace=False))
    pq, ps = routing.permute(*mx.quantize_rowwise(c["x"][np.maximum(src[prow], 0)]), np.where(src[prow] >= 0, np.arange(prow.size), -1))
    assert np.array_equal(host(b.xpq[torch.from_numpy(prow).cuda()]), pq)
    assert np.array_equal(srows(b.xps, K)[prow], ps)

    # W rowwise and columnwise (two experts, sampled rows / columns)
    for e in [empty[0], int(g.integers(0, E))]:
        wr = np.sort(g.choice(N, 16, replace=False))
        oq, os_ = mx.quantize_rowwise(c["w"][e][wr])
        assert np.array_equal(host(b.wq[e])[wr], oq)
        assert np.array_equal(srows(b.wsc, K)[e * N + wr], os_)
        wc = np.sort(g.choice(K, 16, replace=False))
        cq, cs = mx.quantize_rowwise(np.ascontiguousarray(c["w"][e][:, wc].T))
        assert np.array_equal(host(b.wtq[e])[wc], cq)
        assert np.array_equal(srows(b.wtsc, N)[e * K + wc], cs)

    # dY row/col and X columnwise in permuted order (sampled)
    dr = np.sort(g.choice(cap, 32, replace=False))
    oq, os_ = mx.quantize_rowwise(dy_np[dr])
    assert np.array_equal(host(b.dyq)[dr], oq) and np.array_equal(srows(b.dys, N)[dr], os_)
    dc = np.sort(g.choice(N, 8, replace=False))
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(dy_np[:, dc].T))
    assert np.array_equal(host(b.dytq[torch.from_numpy(dc).cuda()]), cq)
    assert np.array_equal(srows(b.dyts, cap)[dc], cs)
    xc = np.sort(g.choice(K, 8, replace=False))
    xg = mx.gather_rows(c["x"][:, xc], src, cap)
    cq, cs = mx.quantize_rowwise(np.ascontiguousarray(xg.T))
    assert np.array_equal(host(b.xtq[torch.from_numpy(xc).cuda()]), cq)
    assert np.array_equal(srows(b.xts, cap)[xc], cs)

    is_bf16 = out_dtype == MX_OUT_BF16
    nsamp = 384

    def grade(name, got, a_rows, b_rows):
        """a_rows, b_rows: bf16 [P, L] operand rows (contraction along L); the
        oracle quantizes them itself and forms the exact dot products."""
        aq, as_ = mx.quantize_rowwise(a_rows)
        bq, bs = mx.quantize_rowwise(b_rows)
        A, B = mx.mx_values(aq, as_), mx.mx_values(bq, bs)
        P = A * B
        C, S = P.sum(-1), np.abs(P).sum(-1)
        ea, eb = tolerance.nominal_exponents(aq, as_), tolerance.nominal_exponents(bq, bs)
        res = tolerance.check(got, C, S, h_fn=lambda i: tolerance.hardware_term(ea[i], eb[i]), out_bf16=is_bf16)
        print(name, res)
        assert res["ok"], (name, res)

    def pick(t, *idx):
        v = t[tuple(torch.from_numpy(np.asarray(i, np.int64)).cuda() for i in idx)].cpu()
        return v.view(torch.int16).numpy().view(np.uint16) if is_bf16 else v.double().numpy()

    grp = np.searchsorted(off, np.arange(cap), side="right") - 1
    real = np.nonzero(src >= 0)[0]

    # fwd: Y[m, n] = X_perm[m] . W_e[n]
    m = g.choice(real, nsamp)
    n = g.integers(0, N, nsamp)
    got = pick(b.y, m, n)
    grade("fwd", got, c["x"][src[m]], c["w"][grp[m], n])

    # dgrad: dX[m, k] = dY[m] . W_e[:, k]
    m = g.choice(real, nsamp)
    k = g.integers(0, K, nsamp)
    got = pick(b.dx, m, k)
    wcol = np.stack([c["w"][grp[mm], :, kk] for mm, kk in zip(m, k)])
    grade("dgrad", got, dy_np[m], wcol)

    # wgrad: dW_e[n, k] = sum over group rows of dY[r, n] X_perm[r, k]
    nonempty = [e for e in range(E) if counts[e] > 0]
    es = g.choice(nonempty, nsamp)
    n = g.integers(0, N, nsamp)
    k = g.integers(0, K, nsamp)
    got = pick(b.dw, es, n, k)
    arows, brows = [], []
    L = int(max(off[e + 1] - off[e] for e in nonempty))
    for e, nn, kk in zip(es, n, k):
        lo, hi = int(off[e]), int(off[e + 1])
        ar = np.zeros(L, np.uint16)
        br = np.zeros(L, np.uint16)
        ar[:hi - lo] = dy_np[lo:hi, nn]
        xr = mx.gather_rows(c["x"][:, kk:kk + 1], src[lo:hi], hi - lo)[:, 0]
        br[:hi - lo] = xr
        arows.append(ar)
        brows.append(br)
    grade("wgrad", got, np.stack(arows), np.stack(brows))
    # empty experts: exact zeros
    for e in empty:
        assert torch.count_nonzero(b.dw[e]) == 0


def test_fused_quantize_permute_matches_full_path(case):
    """The step with the quantize fused into the permute (one gathered pass
    over the bf16 tokens) writes the same bytes as the full path: routing,
    the permuted rowwise MX, the columnwise MX in permuted order, and the
    three GEMM outputs (rows inside the groups)."""
    c, x, w, ids, dy, dy_np, (counts, off, dst, src) = case
    T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
    a = moe.ExpertBuffers(T, K, N, E, topk)
    f = moe.ExpertBuffers(T, K, N, E, topk)
    moe.expert_step(a, x, w, dy, ids)
    moe.fused_expert_step(f, x, w, dy, ids)
    torch.cuda.synchronize()
    hi = int(off[-1])
    for name in ("off", "dst", "src", "xtq", "xts", "wq", "wsc", "dytq", "dyts"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    assert torch.equal(a.xpq[:hi], f.xpq[:hi])
    assert np.array_equal(srows(a.xps, K)[:hi], srows(f.xps, K)[:hi])
    for name in ("y", "dx"):
        assert torch.equal(getattr(a, name)[:hi].view(torch.int16), getattr(f, name)[:hi].view(torch.int16)), name
    assert torch.equal(a.dw.view(torch.int16), f.dw.view(torch.int16))


def grade_tile(name, got, aq, as_, bq, bs, is_bf16, g):
    """Every element of an output tile got [R, Cc] against the exact products
    of operand rows aq [R, L] and bq [Cc, L] (scales [., L/32]); rows are
    aligned so that index 0 starts a k step of the kernel.  Pass rule with H,
    the err/S ceiling, and the instruction-model check on 4096 samples."""
    from gpu_util import MAX_ERR_OVER_S
    A, B = mx.mx_values(aq, as_), mx.mx_values(bq, bs)
    C, S = A @ B.T, np.abs(A) @ np.abs(B).T
    EA, EB = tolerance.nominal_exponents(aq, as_), tolerance.nominal_exponents(bq, bs)
    Cc = bq.shape[0]

    def h_fn(idx):
        out = np.zeros(idx.size)
        for c0 in range(0, idx.size, 2048):
            i, j = np.divmod(idx[c0:c0 + 2048], Cc)
            out[c0:c0 + 2048] = tolerance.hardware_term(EA[i], EB[j])
        return out

    res = tolerance.check(got.ravel(), C.ravel(), S.ravel(), h_fn=h_fn, out_bf16=is_bf16)
    print(name, got.shape, res)
    assert res["ok"], (name, res)
    assert res["max_err_over_S"] <= MAX_ERR_OVER_S, (name, res)
    i = g.integers(0, got.shape[0], 4096)
    j = g.integers(0, Cc, 4096)
    model, bound = tolerance.mfma_model(aq[i], as_[i], bq[j], bs[j])
    rm = tolerance.check_model(got[i, j], model, bound, out_bf16=is_bf16)
    print(name, "model", rm)
    assert rm["ok"], (name, rm)
    return res


@pytest.mark.parametrize("out_dtype", [MX_OUT_BF16, MX_OUT_F32])
def test_expert_step_whole_tiles(case, out_dtype):
    """Whole output tiles of the large workload's GEMMs, with bf16 outputs as
    the benchmark runs them and with fp32 outputs (the accumulation error
    without the bf16 rounding over it), against the oracle on the kernel's
    own MX operand bytes: for fwd and dgrad the last, partly filled 256-row tile of three
    groups (the smallest, the largest, and one next to the empty expert) over
    the first and last 256 output columns; for wgrad a full 256 x 256 dW tile
    of three groups whose rows start inside a 128-row scale panel."""
    c, x, w, ids, dy, dy_np, (counts, off, dst, src) = case
    T, K, N, E, topk, cap = c["T"], c["K"], c["N"], c["E"], c["topk"], c["capacity"]
    b = moe.ExpertBuffers(T, K, N, E, topk, out_dtype=out_dtype)
    moe.expert_step(b, x, w, dy, ids)
    torch.cuda.synchronize()
    g = np.random.default_rng(77)
    is_bf16 = out_dtype == MX_OUT_BF16
    live = [e for e in range(E) if counts[e] > 0]
    empty = [e for e in range(E) if counts[e] == 0]
    nxt = [e for e in live if abs(e - empty[0]) == 1]
    groups = sorted({min(live, key=lambda e: counts[e]), max(live, key=lambda e: counts[e]), nxt[0]})
    xpq, xps = host(b.xpq), srows(b.xps, K)
    dyq, dys = host(b.dyq), srows(b.dys, N)
    wq, ws = host(b.wq), srows(b.wsc, K)
    wtq, wts = host(b.wtq), srows(b.wtsc, N)
    y, dx, dw = host(b.y), host(b.dx), host(b.dw)
    for e in groups:
        lo, hi = int(off[e]), int(off[e + 1])
        r0 = lo + 256 * ((hi - lo - 1) // 256)             # the group's last m tile
        rows = np.arange(r0, hi)
        # the kernel's operand bytes are the oracle's quantize of the inputs
        oq, os_ = mx.quantize_rowwise(mx.gather_rows(c["x"], src[rows], rows.size))
        assert np.array_equal(xpq[rows], oq) and np.array_equal(xps[rows], os_)
        oq, os_ = mx.quantize_rowwise(dy_np[rows])
        assert np.array_equal(dyq[rows], oq) and np.array_equal(dys[rows], os_)
        for cols in (np.arange(0, 256), np.arange(N - 256, N)):
            grade_tile(f"fwd e={e} rows {r0}:{hi} cols {cols[0]}", y[np.ix_(rows, cols)], xpq[rows], xps[rows],
                       wq[e][cols], ws[e * N + cols], is_bf16, g)
        for cols in (np.arange(0, 256), np.arange(K - 256, K)):
            grade_tile(f"dgrad e={e} rows {r0}:{hi} cols {cols[0]}", dx[np.ix_(rows, cols)], dyq[rows], dys[rows],
                       wtq[e][cols], wts[e * K + cols], is_bf16, g)
    # wgrad: groups whose rows start inside a 128-row panel
    dytq, dyts = host(b.dytq), srows(b.dyts, cap)
    xtq, xts = host(b.xtq), srows(b.xts, cap)
    mid = [e for e in live if off[e] % 128 != 0]
    assert len(mid) >= 3
    for e in mid[:3]:
        lo, hi = int(off[e]), int(off[e + 1])
        kb = lo & ~127
        n0 = 256 * int(g.integers(0, N // 256))
        k0 = 256 * int(g.integers(0, K // 256))
        nr, kr = np.arange(n0, n0 + 256), np.arange(k0, k0 + 256)
        aq = dytq[nr, kb:hi].copy()
        bq = xtq[kr, kb:hi].copy()
        aq[:, :lo - kb] = 0
        bq[:, :lo - kb] = 0
        # the kernel's columnwise bytes of this group are the oracle's
        cq, cs = mx.quantize_rowwise(np.ascontiguousarray(dy_np[lo:hi, n0:n0 + 256].T))
        assert np.array_equal(dytq[nr, lo:hi], cq) and np.array_equal(dyts[nr, lo // 32:hi // 32], cs)
        grade_tile(f"wgrad e={e} rows {lo}:{hi} tile ({n0},{k0})", dw[e][np.ix_(nr, kr)], aq,
                   dyts[nr, kb // 32:hi // 32], bq, xts[kr, kb // 32:hi // 32], is_bf16, g)
