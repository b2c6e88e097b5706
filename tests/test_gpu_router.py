"""GPU parity: the router (top-k with softmax weights) and its backward through
the weighted combine, vs the fp64 oracle (oracle/router.py).

* expert ids bit-exact (both sides compare the same fp32 logits);
* weights within 16 fp32 ulps of the exact softmax;
* dw and dlogits within (H/64 + 8) fp32 roundings of their magnitude sums:
  each lane accumulates H/512 x 8 products with fused multiply-adds and the
  wave adds 64 partial sums in 6 levels.
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from oracle import router, routing

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


def check_close(got, exact, S, rel, name):
    err = np.abs(np.asarray(got, np.float64) - exact)
    bound = rel * S + 2.0 ** -126
    bad = err > bound
    print(name, "max err/bound", float((err / bound).max()), "fail", int(bad.sum()))
    assert not bad.any(), (name, np.argwhere(bad)[:5])


@pytest.mark.parametrize("T,E,k", [(1000, 16, 2), (777, 64, 8), (300, 200, 5), (64, 1024, 64), (50, 7, 7), (33, 3, 1)])
def test_route_topk(T, E, k):
    g = np.random.default_rng(T + E + k)
    lg = g.standard_normal((T, E)).astype(np.float32)
    lg[:10, E // 2] = lg[:10, 0]              # exact ties
    lg[10:12] = 1.25                           # a whole row tied
    if E > 4:
        lg[:, 1] = -np.inf                     # an expert nobody may pick (unless k forces it)
    ids, w = mxa.route_topk(dev(lg), k)
    torch.cuda.synchronize()
    oi, ow = router.route_topk(lg, k)
    assert np.array_equal(host(ids), oi)
    check_close(host(w), ow, ow, 2.0 ** -20, "weights")


def test_route_topk_32768_tokens_top8_of_64_full():
    inp = workloads.layer_inputs("cuda:0")
    lg = inp["logits"]
    ids, w = mxa.route_topk(lg, inp["topk"])
    torch.cuda.synchronize()
    oi, ow = router.route_topk(host(lg), inp["topk"])
    assert np.array_equal(host(ids), oi)
    check_close(host(w), ow, ow, 2.0 ** -20, "weights")


@pytest.mark.parametrize("T,H,E,k", [(300, 96, 6, 2), (128, 2048, 64, 8), (77, 544, 9, 3)])
def test_router_bwd(T, H, E, k):
    g = np.random.default_rng(T * H + k)
    lg = g.standard_normal((T, E)).astype(np.float32)
    oi, ow = router.route_topk(lg, k)
    w = ow.astype(np.float32)
    _, off, dst, src = routing.route(oi, E, workloads.capacity(T, k, E))
    rows = src.size
    y = workloads.normal_bf16(g, (rows, H), 1.0, outlier_p=0.01)
    d = workloads.normal_bf16(g, (T, H), 1.0, outlier_p=0.01)
    dw, dl = mxa.router_bwd(dev(d), dev(y), dev(dst), dev(oi), dev(w), E)
    torch.cuda.synchronize()
    edw, sdw, edl, sdl = router.router_bwd(d, y, dst, oi, w, E)
    rel = (H / 64 + 8) * 2.0 ** -24
    check_close(host(dw), edw, sdw, rel, "dw")
    check_close(host(dl), edl, sdl, rel, "dlogits")
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, oi, True, 1)
    assert np.all(host(dl)[~mask] == 0)
