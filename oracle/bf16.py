"""Oracle: the BF16 baseline of the expert step (gather/transpose and the
grouped GEMMs with bf16 operands).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The digest page (Overview, Key Statistics & Figures) measures the MXFP8 MoE
layer against a BF16 one.  The BF16 step computes the same three NT
products as the MXFP8 step, on the bf16 values themselves instead of their
MX encodings:

* fwd:   Y  [M, N]   = X_perm [M, K] . W_e [N, K]^T          (rows grouped)
* dgrad: dX [M, K]   = dY [M, N] . (W_e^T stored [K, N])^T    (rows grouped)
* wgrad: dW_e [N, K] = dY^T [N, M] . X_perm^T [K, M]^T        (contraction grouped)

Every bf16 value is exact in fp64 and so is every product of two of them
(16 significant bits); the oracle multiplies the decoded values per expert
group with an fp64 matmul and also returns S = |A| |B|^T, the per-element
sum of |a_k b_k| the pass rule is measured against.  Group bounds and the
empty-group rules are those of ``oracle.gemm``.
"""

import numpy as np

from .mxfp8 import bf16_to_f64


def gather(x_bits, gather_idx, rows_out):
    """Row gather of a bf16 matrix: output row r is source row gather[r], a
    zero row when gather[r] is negative or past the source; without a
    gather, row r for r < rows and zero after."""
    x = np.asarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    out = np.zeros((rows_out, C), dtype=np.uint16)
    for r in range(rows_out):
        src = r if gather_idx is None else int(gather_idx[r])
        if 0 <= src < R:
            out[r] = x[src]
    return out


def transpose(x_bits):
    """[R, C] -> [C, R] (the layout the GEMM reads along the other axis)."""
    return np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)


def _groups(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(int(off[e]), int(off[e + 1])) for e in range(off.size - 1)]


def grouped_gemm_rows(a_bits, b_bits, offsets, want_abs=True):
    """Row-grouped NT product (fwd and dgrad): a bf16 [M_cap, K], b bf16
    [E, N, K] -> (C, S) fp64 [M_cap, N]; rows outside every group are 0."""
    A = bf16_to_f64(a_bits)
    B = bf16_to_f64(b_bits)
    C = np.zeros((A.shape[0], B.shape[1]))
    S = np.zeros_like(C) if want_abs else None
    for e, (lo, hi) in enumerate(_groups(offsets)):
        if hi > lo:
            C[lo:hi] = A[lo:hi] @ B[e].T
            if want_abs:
                S[lo:hi] = np.abs(A[lo:hi]) @ np.abs(B[e]).T
    return C, S


def grouped_gemm_wgrad(dyt_bits, xt_bits, offsets, want_abs=True):
    """dW_e = dY_e^T X_e over the group's columns: dyt bf16 [N, M_cap], xt
    bf16 [K, M_cap] -> (dW, S) fp64 [E, N, K]; an empty group gives exact 0."""
    DY = bf16_to_f64(dyt_bits)
    X = bf16_to_f64(xt_bits)
    groups = _groups(offsets)
    C = np.zeros((len(groups), DY.shape[0], X.shape[0]))
    S = np.zeros_like(C) if want_abs else None
    for e, (lo, hi) in enumerate(groups):
        if hi > lo:
            C[e] = DY[:, lo:hi] @ X[:, lo:hi].T
            if want_abs:
                S[e] = np.abs(DY[:, lo:hi]) @ np.abs(X[:, lo:hi]).T
    return C, S
