"""The expert step and the SwiGLU layer step captured in a HIP graph
(torch.cuda.CUDAGraph over the C-ABI calls): every replay, with eager work
and synchronizations between replays, reproduces the eager step bit for
bit."""

import numpy as np
import pytest
import torch

import workloads
from mxfp8_block_scaled_07_amd import moe

from gpu_util import dev, host

pytestmark = pytest.mark.gpu


# grouped GEMM outputs: rows past the last group are not written by the
# library (their contents are whatever the buffer held), so only the rows the
# groups own are compared
GROUPED_ROWS = ("y", "dx", "dxp")


def outputs(b, names):
    end = int(host(b.off)[-1])
    out = {}
    for n in names:
        a = host(getattr(b, n)).copy()
        out[n] = a[:end] if n in GROUPED_ROWS and getattr(b, n).shape[0] == b.cap else a
    return out


def test_expert_step_graph_replays_match_eager():
    c = workloads.moe_case(3, 1024, 512, 768, 8, 2, w_std=1.0, outlier_p=0.001, empty_experts=[3])
    T, K, N, E, topk = c["T"], c["K"], c["N"], c["E"], c["topk"]
    x, w, ids = dev(c["x"]), dev(c["w"]), dev(c["expert_ids"])
    eager = moe.ExpertBuffers(T, K, N, E, topk)
    moe.run_stage("quant_x", eager, x, w, None, ids)
    moe.run_stage("permute", eager, x, w, None, ids)
    dy = moe.zero_pad_rows(dev(c["dy_full"][:eager.cap]), eager.src)
    moe.expert_step(eager, x, w, dy, ids)
    torch.cuda.synchronize()
    names = ("off", "src", "xpq", "xps", "wq", "wtq", "dyq", "dytq", "xtq", "y", "dx", "dw")
    ref = outputs(eager, names)
    b = moe.ExpertBuffers(T, K, N, E, topk)
    g = moe.capture(lambda: moe.expert_step(b, x, w, dy, ids))
    for rep in range(3):
        for n in ("y", "dx", "dw", "xpq", "dytq"):
            getattr(b, n).zero_()                       # the replay must rewrite them
        moe.expert_step(eager, x, w, dy, ids)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(b, names)
        for n in names:
            assert np.array_equal(got[n], ref[n]), (rep, n)


def test_layer_step_graph_replays_match_eager():
    inp = workloads.layer_inputs("cuda:0", T=1024, H=256, F=128, E=16, topk=4)
    T, H, F, E, k = inp["T"], inp["H"], inp["F"], inp["E"], inp["topk"]
    args = (inp["x"], inp["w1"], inp["w2"], inp["logits"], inp["dout"])
    eager = moe.LayerBuffers(T, H, F, E, k)
    moe.layer_step(eager, *args)
    torch.cuda.synchronize()
    names = ("ids", "weights", "off", "h", "y", "out", "dw2", "dw1", "dx", "dlogits")
    ref = outputs(eager, names)
    b = moe.LayerBuffers(T, H, F, E, k)
    g = moe.capture(lambda: moe.layer_step(b, *args))
    for rep in range(3):
        for n in ("out", "dw1", "dx", "dlogits"):
            getattr(b, n).zero_()
        moe.layer_step(eager, *args)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(b, names)
        for n in names:
            assert np.array_equal(got[n], ref[n]), (rep, n)
