"""Helpers for the GPU parity tests: numpy <-> device tensors and the
oracle-side tolerance callbacks.  Inputs always come from ``workloads`` or
from the oracle; GPU results are only ever compared, never fed to the oracle."""

import numpy as np
import torch

from oracle import tolerance

DEV = "cuda:0"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    if a.dtype == np.int64:
        return torch.from_numpy(a.astype(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def rows_h_fn(a_q, a_s, b_q, b_s, offsets, N):
    """H for flat indices of a row-grouped [M, N] output."""
    off = np.asarray(offsets)

    def fn(idx):
        m, n = np.divmod(idx, N)
        e = np.searchsorted(off, m, side="right") - 1
        ea = tolerance.nominal_exponents(a_q[m], a_s[m])
        eb = tolerance.nominal_exponents(b_q[e, n], b_s[e, n])
        return tolerance.hardware_term(ea, eb)
    return fn


def wgrad_h_fn(a_q, a_s, b_q, b_s, offsets, N, K):
    """H for flat indices of a wgrad [E, N, K] output."""
    off = np.asarray(offsets)
    EA = tolerance.nominal_exponents(a_q, a_s)
    EB = tolerance.nominal_exponents(b_q, b_s)

    def fn(idx):
        e, rem = np.divmod(idx, N * K)
        n, k = np.divmod(rem, K)
        out = np.zeros(idx.size)
        for ee in np.unique(e):
            sel = e == ee
            lo, hi = int(off[ee]), int(off[ee + 1])
            if hi > lo:
                out[sel] = tolerance.hardware_term(EA[n[sel], lo:hi], EB[k[sel], lo:hi])
        return out
    return fn


def srows(sp, cols):
    """Scale tensor in the kernels' panel layout ([ceil(cols/128), R, 4]
    bytes: panel p, row r holds blocks 4p..4p+3) -> [R, cols/32] row-major,
    the oracle's layout.  Also checks that the pad bytes are zero."""
    a = host(sp) if isinstance(sp, torch.Tensor) else np.asarray(sp)
    P, R, four = a.shape
    assert four == 4 and P == -(-cols // 128), (a.shape, cols)
    full = a.transpose(1, 0, 2).reshape(R, 4 * P)
    nb = cols // 32
    assert not full[:, nb:].any(), "pad bytes of the last scale panel must be zero"
    return np.ascontiguousarray(full[:, :nb])


def spanels(s):
    """[R, nb] row-major scale bytes -> the kernels' panel layout [ceil(nb/4), R, 4]."""
    s = np.asarray(s, np.uint8)
    R, nb = s.shape
    P = -(-nb // 4)
    full = np.zeros((R, 4 * P), np.uint8)
    full[:, :nb] = s
    return np.ascontiguousarray(full.reshape(R, P, 4).transpose(1, 0, 2))


# Ceiling on max |gpu - C| / S for the MXFP8 GEMMs, the largest H / S a run
# can reach: a run loses less than 7 * 2^(emax - 13), and its largest product
# is at least 2^emax with normal codes, 2^(emax - 3) with one subnormal code
# and 2^(emax - 6) with two (subnormal codes count as exponent -6).  Blocks
# beside a x1000 outlier hold subnormal codes, so errors of a few 2^-9 * S
# are legitimate there; the tight check is model_check_* below.
MAX_ERR_OVER_S = 7 * 2.0 ** -7


def model_check_rows(got, a_q, a_s, b_q, b_s, offsets, N, g, n=2048, out_bf16=False):
    """Instruction-model conformance of a row-grouped [M, N] output on n
    sampled elements inside the groups (tolerance.mfma_model)."""
    off = np.asarray(offsets)
    lo, hi = int(off[0]), int(off[-1])
    if hi <= lo:
        return None
    idx = g.integers(lo * N, hi * N, n)
    m, c = np.divmod(idx, N)
    e = np.searchsorted(off, m, side="right") - 1
    model, bound = tolerance.mfma_model(a_q[m], a_s[m], b_q[e, c], b_s[e, c])
    res = tolerance.check_model(np.asarray(got)[m, c], model, bound, out_bf16)
    return res


def model_check_wgrad(got, dyt_q, dyt_s, xt_q, xt_s, offsets, g, n=2048, out_bf16=False):
    """Instruction-model conformance of sampled dW elements: the contraction
    of group e runs over its rows [off[e], off[e+1]) in k steps from the
    128-row panel it starts in, rows outside the group contributing zero."""
    off = np.asarray(offsets)
    E = off.size - 1
    N, K = dyt_q.shape[0], xt_q.shape[0]
    live = [e for e in range(E) if off[e + 1] > off[e]]
    if not live:
        return None
    es = g.choice(live, n)
    ns = g.integers(0, N, n)
    ks = g.integers(0, K, n)
    model = np.zeros(n)
    bound = np.zeros(n)
    for e in np.unique(es):
        sel = es == e
        lo, hi = int(off[e]), int(off[e + 1])
        kb = lo & ~127
        aq = dyt_q[ns[sel], kb:hi].copy()
        bq = xt_q[ks[sel], kb:hi].copy()
        aq[:, :lo - kb] = 0
        bq[:, :lo - kb] = 0
        m_, b_ = tolerance.mfma_model(aq, dyt_s[ns[sel], kb // 32:hi // 32], bq, xt_s[ks[sel], kb // 32:hi // 32])
        model[sel], bound[sel] = m_, b_
    return tolerance.check_model(np.asarray(got)[es, ns, ks], model, bound, out_bf16)
