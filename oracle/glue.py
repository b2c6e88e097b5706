"""Oracle: the glue of the SwiGLU expert FFN around the grouped GEMMs --
SwiGLU with its backward, and the weighted unpermute-combine with its
backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain NumPy in fp64.

The pages run the MoE expert computation in MXFP8 (digest "Key Questions
Answered"; pytorch/ao PR #3203 stacked list and "Next steps": the token
shuffle stays in MXFP8 and the grouped GEMM takes pre-quantized operands) but
give no formula for the layer around the GEMMs.  Readings taken here:

* SwiGLU: the gate/up GEMM output H [R, 2F] holds the gate g in columns
  [0, F) and the up projection u in columns [F, 2F); A = silu(g) * u with
  silu(g) = g * sigmoid(g).  Backward with dA given:
  du = dA * silu(g),  dg = dA * u * sigmoid(g) * (1 + g * (1 - sigmoid(g))).
  The results are bf16 (RNE of the exact value); the requantize that follows
  is the plain MX quantize of those bf16 values (``oracle.mxfp8``).
* Combine: flat routed pair i = t*topk + j sits at permuted row dst_row[i];
  out[t] = sum_j w[t, j] * Y[dst_row[t*topk + j]], rounded to bf16.  Its
  backward scatters the weighted output gradient to the permuted rows:
  dY[dst_row[i]] = w[i] * dOut[t], with the product formed in fp32 (the
  weights' precision) and rounded to bf16; rows no pair maps to are zero.
  The unweighted sum (all w = 1) is the backward of the permute itself:
  dX[t] = sum_j dX_perm[dst_row[t*topk + j]].
"""

import numpy as np

from . import mxfp8


def sigmoid(x):
    """1 / (1 + e^-x) in fp64 (e^-x may overflow to inf for x < -709,
    giving the exact limit 0)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def _split(h_bits, F):
    h = mxfp8.bf16_to_f64(h_bits)
    if h.shape[-1] != 2 * F:
        raise ValueError("swiglu: H must have 2F columns")
    return h[..., :F], h[..., F:]


def swiglu(h_bits, F):
    """Exact (fp64) A = silu(g) * u for H [R, 2F] bf16 bits.  Also returns
    the magnitude |A| that the tolerance is relative to."""
    g, u = _split(h_bits, F)
    a = silu(g) * u
    return a, np.abs(a)


def swiglu_bwd(h_bits, da_bits, F):
    """Exact (fp64) dH = [dg | du] [R, 2F] from H [R, 2F] and dA [R, F] (bf16
    bits), and the per-element magnitude sum S of the terms each result is
    built from (|dA u s| (1 + |g| (1 - s)) for dg, |dA silu(g)| for du)."""
    g, u = _split(h_bits, F)
    da = mxfp8.bf16_to_f64(da_bits)
    s = sigmoid(g)
    dg = da * u * s * (1.0 + g * (1.0 - s))
    du = da * silu(g)
    S = np.concatenate([np.abs(da * u * s) * (1.0 + np.abs(g) * (1.0 - s)), np.abs(du)], axis=-1)
    return np.concatenate([dg, du], axis=-1), S


def combine(y_bits, dst_row, weights, topk):
    """Exact (fp64) out[t] = sum_j w[t, j] * Y[dst_row[t*topk + j]] and
    S = sum_j |w y|.  ``weights`` None means all ones (the unpermute-sum of
    the permute backward).  ``y_bits`` bf16 [M_rows, H]; returns [T, H]."""
    y = mxfp8.bf16_to_f64(y_bits)
    dst = np.asarray(dst_row, dtype=np.int64)
    T = dst.size // topk
    w = (np.ones(dst.size) if weights is None
         else np.asarray(weights, dtype=np.float32).astype(np.float64).ravel())
    out = np.zeros((T, y.shape[1]))
    S = np.zeros((T, y.shape[1]))
    for j in range(topk):
        rows = dst.reshape(T, topk)[:, j]
        wj = w.reshape(T, topk)[:, j:j + 1]
        out += wj * y[rows]
        S += np.abs(wj * y[rows])
    return out, S


def combine_bwd_exact(dout, dst_row, weights, topk, rows):
    """Exact (fp64) scatter dY[dst_row[i]] = w[i] * dOut[i // topk] for real
    values ``dout`` [T, H]; rows that no pair maps to are zero."""
    d = np.asarray(dout, dtype=np.float64)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64).ravel()
    out = np.zeros((rows, d.shape[1]))
    for i in range(dst.size):
        out[dst[i]] = w[i] * d[i // topk]
    return out


def combine_bwd(dout_bits, dst_row, weights, topk, rows):
    """bf16 bits of dY [rows, H]: dY[dst_row[i]] = RNE_bf16(fl32(w[i] *
    dOut[i // topk])), the product rounded once to fp32 (numpy's IEEE
    float32 multiply), then to bf16; unmapped rows are +0."""
    d32 = mxfp8.bf16_to_f64(dout_bits).astype(np.float32)
    dst = np.asarray(dst_row, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float32).ravel()
    out = np.zeros((rows, d32.shape[1]), dtype=np.uint16)
    for i in range(dst.size):
        p = (w[i] * d32[i // topk]).astype(np.float32)
        out[dst[i]] = mxfp8.f64_to_bf16(p.astype(np.float64))
    return out
