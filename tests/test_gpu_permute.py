"""GPU parity: routing metadata and the MXFP8 token permute vs the oracle,
bit-exact (pytorch/ao PR #3203 "Next steps": token shuffle in MXFP8;
TransformerEngine issue #556: codes move together with their scales)."""

import json
import os

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from oracle import mxfp8 as mx
from oracle import routing

from gpu_util import dev, host, spanels, srows

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_permute(ids, E, K=64, seed=0, copy=True, cap=None):
    ids = np.asarray(ids, np.int32).reshape(len(ids), -1)
    T, topk = ids.shape
    cap = T * topk + 31 * E if cap is None else cap
    g = np.random.default_rng(seed)
    xb = workloads.normal_bf16(g, (T, K))
    q, s = mx.quantize_rowwise(xb)
    counts, off, dst, src = routing.route(ids, E, cap)
    qd = dev(q) if copy else None
    sd = dev(spanels(s)) if copy else None
    q_out, s_out, goff, gdst, gsrc = mxa.permute(qd, sd, dev(ids), E, cap)
    torch.cuda.synchronize()
    assert np.array_equal(host(goff), off)
    assert np.array_equal(host(gdst), dst)
    assert np.array_equal(host(gsrc), src)
    if copy:
        oq, os_ = routing.permute(q, s, src)
        assert np.array_equal(host(q_out), oq) and np.array_equal(srows(s_out, K), os_)
    return host(gsrc)


def test_golden_route():
    with open(os.path.join(GOLDEN, "route_small.json")) as fh:
        gd = json.load(fh)
    check_permute(gd["expert_ids"], gd["num_experts"])


def test_workload3_routing_full_width():
    """8192 tokens, top-2 of 16 experts with one empty expert, 5120 columns."""
    c = workloads.moe_case(3, 8192, 32, 32, 16, 2, empty_experts=[5], with_dy=False)
    ids = c["expert_ids"]
    assert not np.any(ids == 5)
    check_permute(ids, 16, K=5120, seed=3)


def test_top8_of_64_routing():
    c = workloads.moe_case(5, 32768, 32, 32, 64, 8, with_dy=False)
    check_permute(c["expert_ids"], 64, K=256, seed=5)


@pytest.mark.parametrize("T,topk,E", [(1, 1, 1), (5, 3, 2), (63, 2, 7), (4097, 1, 3), (3000, 2, 300), (100, 4, 1),
                                      (5000, 2, 2048),      # above 1024 experts: 4096-pair routing tiles
                                      (3000, 1, 16384),     # the largest expert count (most experts empty)
                                      (300, 8, 16),         # the most destinations the copy reads directly
                                      (250, 9, 16)])        # one more: destinations staged through LDS
def test_edge_shapes(T, topk, E):
    g = np.random.default_rng(T * 7 + E)
    ids = g.integers(0, E, (T, topk))
    check_permute(ids, E, K=32 * int(g.integers(1, 4)), seed=T)


@pytest.mark.parametrize("T,topk,E", [(300, 3, 7), (20000, 2, 9), (2000, 12, 600)])
def test_out_of_range_ids_are_ignored(T, topk, E):
    """Pairs whose expert id is negative or >= E get dst_row -1, count in no
    group and are not copied; the valid pairs keep their flat-order ranks.
    Expected values: the oracle's routing with one extra expert E that
    collects the invalid pairs (it sorts after every real expert, so experts
    0..E-1 get the same offsets and rows as with those pairs dropped)."""
    g = np.random.default_rng(T + E)
    ids = g.integers(0, E, (T, topk)).astype(np.int32)
    flat = ids.reshape(-1)
    flat[::29] = -1
    flat[7::41] = E + 5
    bad = (flat < 0) | (flat >= E)
    cap = T * topk + 31 * E
    _, off, dst, src = routing.route(np.where(bad, E, flat).reshape(T, topk), E + 1, cap + 31)
    off = off[:E + 1]
    dst = np.where(bad, -1, dst)
    src = src[:cap].copy()
    src[off[E]:] = -1
    K = 64
    xb = workloads.normal_bf16(g, (T, K))
    q, s = mx.quantize_rowwise(xb)
    q_out, s_out, goff, gdst, gsrc = mxa.permute(dev(q), dev(spanels(s)), dev(ids), E, cap)
    torch.cuda.synchronize()
    assert np.array_equal(host(goff), off)
    assert np.array_equal(host(gdst), dst)
    assert np.array_equal(host(gsrc), src)
    oq, os_ = routing.permute(q, s, src)
    assert np.array_equal(host(q_out), oq) and np.array_equal(srows(s_out, K), os_)


def test_no_tokens():
    """A call with no tokens: every group is empty, every row of the
    capacity is a pad row (src_row -1, zero codes and scales)."""
    E, K, cap = 4, 64, 4 * 31 + 40
    ids = torch.zeros((0, 2), dtype=torch.int32, device="cuda:0")
    # one-row sources: with no tokens nothing is read from them (an empty
    # tensor may have a null data pointer, which the copy rejects)
    q = torch.zeros((1, K), dtype=torch.uint8, device="cuda:0")
    s = torch.zeros(mxa.scale_shape(1, K), dtype=torch.uint8, device="cuda:0")
    q_out, s_out, goff, gdst, gsrc = mxa.permute(q, s, ids, E, cap)
    torch.cuda.synchronize()
    assert np.array_equal(host(goff), np.zeros(E + 1))
    assert host(gdst).size == 0
    assert np.array_equal(host(gsrc), np.full(cap, -1))
    assert not host(q_out).any() and not host(s_out).any()


def test_rows_wider_than_one_block():
    """Rows of 16416 codes (1026 16-byte chunks, 129 scale panels): the copy's
    1024-thread blocks loop over the chunks."""
    g = np.random.default_rng(11)
    check_permute(g.integers(0, 5, (70, 2)), 5, K=16416, seed=11)


def test_all_tokens_one_expert_and_duplicates():
    ids = np.zeros((300, 2), np.int32)
    ids[::3, 1] = 2
    check_permute(ids, 4)


def test_metadata_only_and_extra_capacity():
    g = np.random.default_rng(2)
    ids = g.integers(0, 6, (500, 2))
    check_permute(ids, 6, copy=False)
    check_permute(ids, 6, cap=500 * 2 + 31 * 6 + 77)


def test_permute_deterministic():
    c = workloads.moe_case(3, 8192, 32, 32, 16, 2, with_dy=False)
    a = check_permute(c["expert_ids"], 16, K=128)
    b = check_permute(c["expert_ids"], 16, K=128)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T,topk,E", [(200, 70, 80), (40, 129, 5)])
def test_topk_above_64(T, topk, E):
    """More routed copies per token than the permute's 64-slot table holds:
    the slots are copied in chunks of 64."""
    g = np.random.default_rng(T + topk)
    check_permute(g.integers(0, E, (T, topk)), E, K=96, seed=topk)


def test_permute_rejects_misaligned_codes():
    T, K, E, topk = 64, 64, 2, 2
    ids = torch.zeros((T, topk), dtype=torch.int32, device="cuda:0")
    cap = T * topk + 31 * E
    buf = torch.zeros(T * K + 16, dtype=torch.uint8, device="cuda:0")
    q = buf[8:8 + T * K]                                  # 8-byte aligned only
    s = torch.zeros(mxa.scale_shape(T, K), dtype=torch.uint8, device="cuda:0")
    q_out = torch.zeros((cap, K), dtype=torch.uint8, device="cuda:0")
    s_out = torch.zeros(mxa.scale_shape(cap, K), dtype=torch.uint8, device="cuda:0")
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda:0")
    dst = torch.zeros(T * topk, dtype=torch.int32, device="cuda:0")
    src = torch.zeros(cap, dtype=torch.int32, device="cuda:0")
    wsb = mxa.mx_permute_workspace_size(T, topk, E)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(mxa.MXError):
        mxa.mx_permute(q, s, T, K, ids, topk, E, cap, q_out, s_out, off, dst, src, ws, wsb)
