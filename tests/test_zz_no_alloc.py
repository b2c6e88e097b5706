"""mx_permute_noalloc (the permute for callers that cannot allocate device
memory) against mx_permute, through the C ABI: routing metadata and permuted
MX bytes bit-identical, on two calls in a row (the second smaller, so stale
routing tables of the first call in the shared device array would show), and
oversized requests rejected before any launch."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads

pytestmark = pytest.mark.gpu


def _case(seed, T, K, E, topk, empty=()):
    g = np.random.default_rng(seed)
    logits = g.standard_normal((T, E)).astype(np.float32)
    for e in empty:
        logits[:, e] = -np.inf
    ids, _ = workloads.topk_route(logits, topk)
    q = torch.from_numpy(g.integers(0, 256, (T, K), dtype=np.uint8)).cuda()
    s = torch.from_numpy(g.integers(0, 256, mxa.scale_shape(T, K), dtype=np.uint8)).cuda()
    return q, s, torch.from_numpy(ids.astype(np.int32)).cuda()


def _outputs(T, K, E, topk):
    cap = -(-(T * topk + 31 * E) // 32) * 32
    dev = "cuda:0"
    return cap, dict(q=torch.full((cap, K), 0xAB, dtype=torch.uint8, device=dev),
                     s=torch.full(mxa.scale_shape(cap, K), 0xCD, dtype=torch.uint8, device=dev),
                     off=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                     dst=torch.full((T * topk,), -7, dtype=torch.int32, device=dev),
                     src=torch.full((cap,), -7, dtype=torch.int32, device=dev))


def _both(T, K, E, topk, seed, empty=()):
    q, s, ids = _case(seed, T, K, E, topk, empty)
    cap, a = _outputs(T, K, E, topk)
    _, b = _outputs(T, K, E, topk)
    wsb = mxa.mx_permute_workspace_size(T, topk, E)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda:0")
    mxa.mx_permute(q, s, T, K, ids, topk, E, cap, a["q"], a["s"], a["off"], a["dst"], a["src"], ws, wsb)
    mxa.mx_permute_noalloc(q, s, T, K, ids, topk, E, cap, b["q"], b["s"], b["off"], b["dst"], b["src"])
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), (T, K, E, topk, name)
    return a


def test_noalloc_permute_matches_permute_twice():
    # a large call (top-8 of 64 experts) that fills many routing tiles, then a
    # smaller one (top-2 of 16, one expert empty) that reuses the same tables
    first = _both(4096, 512, 64, 8, 1)
    assert int(first["off"][-1]) >= 4096 * 8
    second = _both(1000, 256, 16, 2, 2, empty=(5,))
    off = second["off"].cpu().numpy()
    assert off[6] == off[5]                       # the empty expert
    # metadata only (no tensors), and a call with no tokens
    cap, a = _outputs(300, 0, 8, 1)
    _, b = _outputs(300, 0, 8, 1)
    ids = torch.from_numpy(np.arange(300, dtype=np.int32)[:, None] % 8).cuda()
    ws = torch.empty(mxa.mx_permute_workspace_size(300, 1, 8), dtype=torch.uint8, device="cuda:0")
    mxa.mx_permute(None, None, 300, 0, ids, 1, 8, cap, None, None, a["off"], a["dst"], a["src"], ws, ws.numel())
    mxa.mx_permute_noalloc(None, None, 300, 0, ids, 1, 8, cap, None, None, b["off"], b["dst"], b["src"])
    torch.cuda.synchronize()
    for name in ("off", "dst", "src"):
        assert torch.equal(a[name], b[name]), name


def test_noalloc_permute_rejects_oversized_requests():
    # 16384 experts x 256k pairs needs far more than the built-in scratch
    T, topk, E = 1 << 18, 1, 16384
    assert mxa.mx_permute_workspace_size(T, topk, E) > mxa.lib().mx_permute_workspace_size(1, 1, 1)
    P = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    with pytest.raises(mxa.MXError, match="MX_EUNSUPPORTED"):
        mxa.mx_permute_noalloc(None, None, T, 0, P, topk, E, T + 31 * E, None, None, P, P, P)
