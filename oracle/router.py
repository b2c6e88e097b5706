"""Oracle: the router in front of the token shuffle -- top-k expert choice with
softmax weights -- and its backward through the weighted combine.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain NumPy in fp64.

The pages name the MoE layer (digest "Overview": MoE training in MXFP8) but
give no router formula.  The reading taken here, the one the routing of the
workloads uses:

* each token's experts are the k largest logits, ties to the lower expert id;
* the combine weights are the softmax of the k chosen logits (renormalised
  over the chosen experts, not over all E);
* backward: with out[t] = sum_j w[t,j] Y[dst_row[t k + j]], the weight
  gradient is dw[t,j] = <dOut[t], Y[dst_row[t k + j]]>, and the softmax
  backward gives d logit[t, e_j] = w_j (dw_j - sum_i w_i dw_i) for the chosen
  experts e_j and 0 for the others.
"""

import numpy as np

from . import mxfp8


def route_topk(logits, topk):
    """(expert ids int64 [T, k], weights fp64 [T, k]) for fp32 logits [T, E]:
    ids in order of decreasing logit, equal logits by increasing id."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = lg.shape
    if not 1 <= topk <= E:
        raise ValueError("route_topk: need 1 <= topk <= E")
    ids = np.zeros((T, topk), dtype=np.int64)
    w = np.zeros((T, topk))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:topk]
        ids[t] = order
        z = lg[t, order]
        ez = np.exp(z - z.max())
        w[t] = ez / ez.sum()
    return ids, w


def router_bwd(dout_bits, y_bits, dst_row, expert_ids, weights, num_experts):
    """Exact (fp64) weight gradient dw [T, k] and logit gradient dlogits
    [T, E], with the magnitude sums the tolerance is relative to:
    S_dw[t,j] = sum_h |dOut[t,h] Y[r,h]| and
    S_dl[t,e_j] = w_j (S_dw[t,j] + sum_i w_i S_dw[t,i])."""
    d = mxfp8.bf16_to_f64(dout_bits)
    y = mxfp8.bf16_to_f64(y_bits)
    ids = np.asarray(expert_ids, dtype=np.int64)
    T, k = ids.shape
    w = np.asarray(weights, dtype=np.float64).reshape(T, k)   # fp32 weights convert exactly
    rows = np.asarray(dst_row, dtype=np.int64).reshape(T, k)
    dw = np.zeros((T, k))
    sdw = np.zeros((T, k))
    for j in range(k):
        yr = y[rows[:, j]]
        dw[:, j] = np.sum(d * yr, axis=1)
        sdw[:, j] = np.sum(np.abs(d * yr), axis=1)
    inner = np.sum(w * dw, axis=1, keepdims=True)
    dsel = w * (dw - inner)
    ssel = w * (sdw + np.sum(w * sdw, axis=1, keepdims=True))
    dl = np.zeros((T, num_experts))
    sl = np.zeros((T, num_experts))
    for j in range(k):
        np.add.at(dl, (np.arange(T), ids[:, j]), dsel[:, j])
        np.add.at(sl, (np.arange(T), ids[:, j]), ssel[:, j])
    return dw, sdw, dl, sl
