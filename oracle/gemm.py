"""Oracle: block-scaled grouped GEMMs for the expert forward, dgrad and wgrad.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

pytorch/ao PR #3203, "Next steps": the scaled grouped GEMM takes
pre-quantized MXFP8 tensors (codes plus scales).  The digest page ("Key
Questions Answered") puts the block scales inside the matrix multiply.  The
oracle decodes both operands exactly to fp64 (E4M3 value times 2^(byte-127))
and multiplies them per expert group with an fp64 matmul, so the result is
the exact sum up to fp64 rounding (about 1e-16 relative).  It also returns
S = |A| |B|^T, the per-element sum of |a_k b_k| that the tolerance is
measured against.

All three products are "NT": C[m, n] = sum_k A[m, k] B[n, k] with both
operands contiguous along the contraction axis k (blocks of 32 along k).

* fwd:   Y  [M, N]   = X_perm [M, K] . W_e [N, K]^T        (rows grouped)
* dgrad: dX [M, K]   = dY [M, N] . (W_e^T stored [K, N])^T  (rows grouped)
* wgrad: dW_e [N, K] = dY^T [N, M] . X^T [K, M]^T           (contraction grouped)

Group e owns rows (fwd, dgrad) or contraction columns (wgrad)
[offsets[e], offsets[e+1]).  An expert with no rows gives no output rows in
fwd/dgrad and an exact zero dW_e in wgrad.
"""

import numpy as np

from . import mxfp8


def _groups(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(int(off[e]), int(off[e + 1])) for e in range(off.size - 1)]


def grouped_gemm_rows(a_q, a_s, b_q, b_s, offsets, want_abs=True):
    """Row-grouped NT product (forward and dgrad).

    a: [M_cap, K] codes with [M_cap, K/32] scales; b: [E, N, K] codes with
    [E, N, K/32] scales.  Returns (C, S), fp64 [M_cap, N]; rows outside every
    group are 0.
    """
    A = mxfp8.mx_values(a_q, a_s)
    Bv = mxfp8.mx_values(b_q, b_s)
    M = A.shape[0]
    N = Bv.shape[1]
    C = np.zeros((M, N))
    S = np.zeros((M, N)) if want_abs else None
    for e, (lo, hi) in enumerate(_groups(offsets)):
        if hi > lo:
            C[lo:hi] = A[lo:hi] @ Bv[e].T
            if want_abs:
                S[lo:hi] = np.abs(A[lo:hi]) @ np.abs(Bv[e]).T
    return C, S


def grouped_gemm_fwd(x_q, x_s, w_q, w_s, offsets, want_abs=True):
    """Expert forward Y = X_perm . W_e^T per group (see module docstring)."""
    return grouped_gemm_rows(x_q, x_s, w_q, w_s, offsets, want_abs)


def grouped_gemm_dgrad(dy_q, dy_s, wt_q, wt_s, offsets, want_abs=True):
    """Expert dgrad dX = dY . W_e per group; W_e enters as its columnwise
    quantization stored transposed, [E, K, N]."""
    return grouped_gemm_rows(dy_q, dy_s, wt_q, wt_s, offsets, want_abs)


def grouped_gemm_wgrad(dyt_q, dyt_s, xt_q, xt_s, offsets, want_abs=True):
    """Expert wgrad dW_e = dY_e^T . X_e per group, contracting over the group's
    token rows.  dyt: [N, M_cap] codes ([N, M_cap/32] scales), xt: [K, M_cap]
    codes; offsets are multiples of 32.  Returns (dW, S) fp64 [E, N, K]."""
    DY = mxfp8.mx_values(dyt_q, dyt_s)
    X = mxfp8.mx_values(xt_q, xt_s)
    groups = _groups(offsets)
    E = len(groups)
    N, K = DY.shape[0], X.shape[0]
    C = np.zeros((E, N, K))
    S = np.zeros((E, N, K)) if want_abs else None
    for e, (lo, hi) in enumerate(groups):
        if hi > lo:
            C[e] = DY[:, lo:hi] @ X[:, lo:hi].T
            if want_abs:
                S[e] = np.abs(DY[:, lo:hi]) @ np.abs(X[:, lo:hi]).T
    return C, S


def dot_rows(a_vals, b_vals):
    """Exact-in-fp64 per-pair dot products and |.| sums for sampled outputs:
    a_vals, b_vals [P, K] fp64 -> (sum_k a b, sum_k |a b|)."""
    p = np.asarray(a_vals) * np.asarray(b_vals)
    return p.sum(axis=-1), np.abs(p).sum(axis=-1)
