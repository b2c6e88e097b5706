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
