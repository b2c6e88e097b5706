"""Oracle: routing metadata and the MXFP8 token permute.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

pytorch/ao PR #3203, "Next steps", asks for a token shuffle that keeps the
tokens in MXFP8 (no dequantize before the grouped GEMM);
NVIDIA/TransformerEngine issue #556, first maintainer reply, notes that moving
fp8 data is plain byte movement as long as the scales travel with the bytes.
So the permute copies each token's E4M3 codes and its E8M0 scales together,
unchanged.

Readings taken (the pages only name the kernel):

* routed rows are the flat pairs i = t*topk + j of an ``expert_ids[T, topk]``
  table; a duplicated expert id in one token counts as two assignments;
* each expert's group is padded with zero rows to a multiple of 32 so that a
  columnwise 32-row block never straddles two experts; groups are laid out
  in expert order;
* within a group rows keep their flat order (stable); any order that keeps
  the grouping is a valid MoE permutation, so this pins one of them.
"""

import numpy as np

BLOCK = 32


def route(expert_ids, num_experts, capacity_rows=None):
    """Routing metadata for a flat list of (token, slot) -> expert choices.

    Returns ``counts`` [E], ``offsets`` [E+1] (padded exclusive prefix sum,
    every entry a multiple of 32), ``dst_row`` [T*topk] (the permuted row of
    flat pair i) and ``src_row`` [capacity_rows] (the source token of each
    permuted row, -1 for pad rows and for rows past the last group).
    """
    ids = np.asarray(expert_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("route: expert id out of range")
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    padded = (counts + BLOCK - 1) // BLOCK * BLOCK
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    if capacity_rows is None:
        capacity_rows = T * topk + (BLOCK - 1) * num_experts
    if offsets[-1] > capacity_rows:
        raise ValueError("route: capacity_rows too small")
    dst_row = np.zeros(flat.size, dtype=np.int64)
    next_free = offsets[:-1].copy()
    for i, e in enumerate(flat):          # stable: flat order within each expert
        dst_row[i] = next_free[e]
        next_free[e] += 1
    src_row = np.full(capacity_rows, -1, dtype=np.int64)
    src_row[dst_row] = np.arange(flat.size) // topk
    return counts, offsets, dst_row, src_row


def permute(q, s, src_row):
    """Permuted MX rows: row r of the output is row ``src_row[r]`` of (q, s),
    codes and scales together; rows with ``src_row[r] < 0`` are all-zero
    codes (0x00) with zero scale bytes (0x00)."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    src = np.asarray(src_row, dtype=np.int64)
    qo = np.zeros((src.size, q.shape[1]), dtype=np.uint8)
    so = np.zeros((src.size, s.shape[1]), dtype=np.uint8)
    ok = src >= 0
    qo[ok] = q[src[ok]]
    so[ok] = s[src[ok]]
    return qo, so
