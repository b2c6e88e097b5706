"""GPU parity: block-scaled grouped GEMMs (fwd, dgrad, wgrad) vs the fp64
oracle, element by element, under the pass rule of oracle/tolerance.py
(digest "Key Questions Answered": block-scaled MMA; pytorch/ao PR #3203 "Next
steps": grouped GEMM on pre-quantized tensors)."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_07_amd as mxa
import workloads
from oracle import gemm as og
from oracle import mxfp8 as mx
from oracle import routing, tolerance

from gpu_util import MAX_ERR_OVER_S, dev, host, model_check_rows, model_check_wgrad, rows_h_fn, spanels, wgrad_h_fn

pytestmark = pytest.mark.gpu


def run_rows(kind, a_q, a_s, b_q, b_s, off, N, K, out_dtype, sentinel=True):
    M = a_q.shape[0]
    E = b_q.shape[0]
    dt = torch.float32 if out_dtype == mxa.MX_OUT_F32 else torch.bfloat16
    out = torch.full((M, N), 7.0 if sentinel else 0.0, dtype=dt, device="cuda:0")
    fn = mxa.mx_grouped_gemm_fwd if kind == "fwd" else mxa.mx_grouped_gemm_dgrad
    fn(dev(a_q), dev(spanels(a_s)), dev(b_q), dev(spanels(b_s.reshape(-1, b_s.shape[-1]))),
       dev(np.asarray(off, np.int32)), E, M, N, K, out, out_dtype)
    torch.cuda.synchronize()
    return host(out) if out_dtype == mxa.MX_OUT_BF16 else host(out).astype(np.float64)


def check_rows(kind, a_q, a_s, b_q, b_s, off, out_dtype):
    N, K = b_q.shape[1], b_q.shape[2]
    got = run_rows(kind, a_q, a_s, b_q, b_s, off, N, K, out_dtype)
    C, S = og.grouped_gemm_rows(a_q, a_s, b_q, b_s, off)
    lo, hi = int(off[0]), int(off[-1])
    res = tolerance.check(got[lo:hi], C[lo:hi], S[lo:hi], h_fn=lambda i: rows_h_fn(
        a_q, a_s, b_q, b_s, off, N)(i + lo * N), out_bf16=out_dtype == mxa.MX_OUT_BF16)
    print(kind, res)
    assert res["ok"], res
    assert res["max_err_over_S"] <= MAX_ERR_OVER_S, res
    rm = model_check_rows(got, a_q, a_s, b_q, b_s, off, N, np.random.default_rng(N + K),
                          out_bf16=out_dtype == mxa.MX_OUT_BF16)
    print(kind, "model", rm)
    assert rm is None or rm["ok"], rm
    # rows outside every group are left untouched
    outside = np.r_[0:lo, hi:a_q.shape[0]]
    if outside.size:
        sent = got[outside]
        if out_dtype == mxa.MX_OUT_BF16:
            assert np.all(sent == 0x40E0)
        else:
            assert np.all(sent == 7.0)
    return res


def mx_rows(g, shape, std=1.0, outlier_p=0.0):
    xb = workloads.normal_bf16(g, shape, std, outlier_p)
    return mx.quantize_rowwise(xb)


def test_workload1_forward_fp32():
    c = workloads.config(1)
    ids = c["expert_ids"]
    counts, off, dst, src = routing.route(ids, c["E"], c["T"])
    a_q, a_s = routing.permute(*mx.quantize_rowwise(c["x"]), src)
    w_q, w_s = mx.quantize_rowwise(c["w"])
    check_rows("fwd", a_q, a_s, w_q, w_s, off, mxa.MX_OUT_F32)


@pytest.mark.parametrize("out_dtype", [mxa.MX_OUT_F32, mxa.MX_OUT_BF16])
def test_workload2_fwd_dgrad_wgrad(out_dtype):
    c = workloads.config(2)
    T, K, N, E = c["T"], c["K"], c["N"], c["E"]
    cap = c["capacity"]
    counts, off, dst, src = routing.route(c["expert_ids"], E, cap)
    xq, xs = mx.quantize_rowwise(c["x"])
    a_q, a_s = routing.permute(xq, xs, src)
    w_q, w_s = mx.quantize_rowwise(c["w"])
    check_rows("fwd", a_q, a_s, w_q, w_s, off, out_dtype)
    wt = [mx.quantize_colwise(c["w"][e]) for e in range(E)]
    wt_q, wt_s = np.stack([t[0] for t in wt]), np.stack([t[1] for t in wt])
    dy = c["dy_full"].copy()
    dy[src < 0] = 0
    dy_q, dy_s = mx.quantize_rowwise(dy)
    check_rows("dgrad", dy_q, dy_s, wt_q, wt_s, off, out_dtype)
    dyt_q, dyt_s = mx.quantize_colwise(dy)
    xt_q, xt_s = mx.quantize_colwise(c["x"], rows_out=cap, gather=src)
    check_wgrad(dyt_q, dyt_s, xt_q, xt_s, off, out_dtype)


def check_wgrad(dyt_q, dyt_s, xt_q, xt_s, off, out_dtype):
    N, cap = dyt_q.shape
    K = xt_q.shape[0]
    E = len(off) - 1
    dt = torch.float32 if out_dtype == mxa.MX_OUT_F32 else torch.bfloat16
    dw = torch.full((E, N, K), 7.0, dtype=dt, device="cuda:0")
    mxa.mx_grouped_gemm_wgrad(dev(dyt_q), dev(spanels(dyt_s)), dev(xt_q), dev(spanels(xt_s)),
                              dev(np.asarray(off, np.int32)), E, cap,
                              N, K, dw, out_dtype)
    torch.cuda.synchronize()
    got = host(dw) if out_dtype == mxa.MX_OUT_BF16 else host(dw).astype(np.float64)
    C, S = og.grouped_gemm_wgrad(dyt_q, dyt_s, xt_q, xt_s, off)
    res = tolerance.check(got, C, S, h_fn=wgrad_h_fn(dyt_q, dyt_s, xt_q, xt_s, off, N, K),
                          out_bf16=out_dtype == mxa.MX_OUT_BF16)
    print("wgrad", res)
    assert res["ok"], res
    assert res["max_err_over_S"] <= MAX_ERR_OVER_S, res
    rm = model_check_wgrad(got, dyt_q, dyt_s, xt_q, xt_s, off, np.random.default_rng(N + K),
                           out_bf16=out_dtype == mxa.MX_OUT_BF16)
    print("wgrad model", rm)
    assert rm is None or rm["ok"], rm
    for e in range(E):
        if off[e + 1] == off[e]:
            z = got[e].astype(np.float64) if out_dtype == mxa.MX_OUT_F32 else got[e]
            assert np.all(z == 0)
    return res


@pytest.mark.parametrize("sizes,N,K", [
    ([1, 31, 0, 64, 200], 96, 160),          # group of 1 row, 31 rows, an empty group, N and K tails
    ([0, 0, 3], 32, 32),                     # single 32-block contraction, leading empty groups
    ([300], 256, 384),                       # one expert
    ([129, 0, 127, 1], 160, 4224),           # M tiles split across groups, long K
])
def test_edge_shapes_rows(sizes, N, K):
    g = np.random.default_rng(sum(sizes) + N + K)
    E = len(sizes)
    ids = workloads.ids_from_sizes(sizes)
    T = int(sum(sizes))
    counts, off, dst, src = routing.route(ids, E)
    a_q, a_s = routing.permute(*mx_rows(g, (T, K), 1.0, 0.01), src)
    b_q, b_s = mx_rows(g, (E * N, K), 0.02)
    b_q, b_s = b_q.reshape(E, N, K), b_s.reshape(E, N, K // 32)
    for dt in (mxa.MX_OUT_F32, mxa.MX_OUT_BF16):
        check_rows("fwd", a_q, a_s, b_q, b_s, off, dt)


def test_rows_outside_groups_untouched():
    g = np.random.default_rng(77)
    M, N, K = 320, 64, 128
    a_q, a_s = mx_rows(g, (M, K))
    b_q, b_s = mx_rows(g, (2 * N, K))
    b_q, b_s = b_q.reshape(2, N, K), b_s.reshape(2, N, K // 32)
    check_rows("fwd", a_q, a_s, b_q, b_s, np.array([32, 96, 224]), mxa.MX_OUT_F32)


@pytest.mark.parametrize("lens,N,K", [([32, 64, 0, 96, 160], 96, 160), ([0, 0], 64, 32), ([4096], 128, 256),
                                      ([32, 1056, 0, 480], 192, 288)])
def test_edge_shapes_wgrad(lens, N, K):
    g = np.random.default_rng(sum(lens) + N)
    off = np.concatenate([[0], np.cumsum(lens)])
    cap = int(off[-1]) + 32
    dyt_q, dyt_s = mx_rows(g, (N, cap), 1.0, 0.01)
    xt_q, xt_s = mx_rows(g, (K, cap))
    for dt in (mxa.MX_OUT_F32, mxa.MX_OUT_BF16):
        check_wgrad(dyt_q, dyt_s, xt_q, xt_s, off, dt)


@pytest.mark.parametrize("lens,N,K", [
    ([6016, 0, 32, 0, 0, 2048, 64, 0, 960], 512, 512),   # XCD range bounds inside the large group's tiles
    ([0, 0, 0, 0], 256, 256),                            # all empty: every tile stores zeros
    ([4096, 32], 96, 64),                                # fewer tiles than workgroups
])
def test_wgrad_work_split_extremes(lens, N, K):
    """The wgrad tiles are split among XCDs by work (k steps per tile);
    skewed and empty groups still give every dW element exactly once."""
    g = np.random.default_rng(len(lens) + N + K)
    off = np.concatenate([[0], np.cumsum(lens)])
    cap = int(off[-1]) + 32
    dyt_q, dyt_s = mx_rows(g, (N, cap), 1.0, 0.01)
    xt_q, xt_s = mx_rows(g, (K, cap))
    check_wgrad(dyt_q, dyt_s, xt_q, xt_s, off, mxa.MX_OUT_F32)


def test_max_groups_fwd_and_wgrad():
    """2048 groups, the most one call takes, most of them tiny or empty:
    forward over ragged groups of 0 to 64 rows, wgrad over groups of 0, 32
    or 64 rows; both compared in full."""
    g = np.random.default_rng(2048)
    E, N, K = 2048, 64, 96
    sizes = g.choice([0, 0, 1, 17, 32, 45, 64], E)
    ids = workloads.ids_from_sizes(sizes)
    counts, off, dst, src = routing.route(ids, E)
    a_q, a_s = routing.permute(*mx_rows(g, (int(sizes.sum()), K), 1.0, 0.01), src)
    b_q, b_s = mx_rows(g, (E * N, K), 0.02)
    b_q, b_s = b_q.reshape(E, N, K), b_s.reshape(E, N, K // 32)
    check_rows("fwd", a_q, a_s, b_q, b_s, off, mxa.MX_OUT_F32)
    woff = np.concatenate([[0], np.cumsum(g.choice([0, 32, 64], E))])
    cap = int(woff[-1]) + 32
    dyt_q, dyt_s = mx_rows(g, (N, cap), 1.0, 0.01)
    xt_q, xt_s = mx_rows(g, (K, cap))
    check_wgrad(dyt_q, dyt_s, xt_q, xt_s, woff, mxa.MX_OUT_F32)


def test_wgrad_nan_block_stays_in_its_group():
    """A NaN block (scale byte 0xFF) in one group's rows of dY^T or X^T makes
    only that group's matching dW row or column NaN: the groups that share its
    128-row scale panel are unaffected (groups start at multiples of 32)."""
    g = np.random.default_rng(31)
    off = np.array([0, 96, 224, 320])
    E, cap, N, K = 3, 352, 64, 96
    dyt_q, dyt_s = mx_rows(g, (N, cap), 1.0, 0.01)
    xt_q, xt_s = mx_rows(g, (K, cap))
    dyt_s[5, 2] = 0xFF    # rows 64..95: group 0, panel 0 shared with group 1
    dyt_s[9, 7] = 0xFF    # rows 224..255: group 2, panel 1 shared with group 1
    xt_s[3, 3] = 0xFF     # rows 96..127: group 1, panel 0 shared with group 0
    nan = np.zeros((E, N, K), bool)
    nan[0, 5, :] = True
    nan[2, 9, :] = True
    nan[1, :, 3] = True
    C, S = og.grouped_gemm_wgrad(dyt_q, dyt_s, xt_q, xt_s, off)
    assert np.all(np.isnan(C[nan])) and np.all(np.isfinite(C[~nan]))
    dw = torch.full((E, N, K), 7.0, dtype=torch.float32, device="cuda:0")
    mxa.mx_grouped_gemm_wgrad(dev(dyt_q), dev(spanels(dyt_s)), dev(xt_q), dev(spanels(xt_s)),
                              dev(off.astype(np.int32)), E, cap, N, K, dw, mxa.MX_OUT_F32)
    torch.cuda.synchronize()
    got = host(dw).astype(np.float64)
    assert np.all(np.isnan(got[nan]))
    got[nan] = C[nan] = S[nan] = 0.0
    res = tolerance.check(got, C, S, h_fn=wgrad_h_fn(dyt_q, dyt_s, xt_q, xt_s, off, N, K))
    print("wgrad nan", res)
    assert res["ok"], res


def test_gemm_deterministic():
    g = np.random.default_rng(5)
    a_q, a_s = mx_rows(g, (256, 512))
    b_q, b_s = mx_rows(g, (256, 512))
    b_q, b_s = b_q.reshape(1, 256, 512), b_s.reshape(1, 256, 16)
    r1 = run_rows("fwd", a_q, a_s, b_q, b_s, [0, 256], 256, 512, mxa.MX_OUT_F32)
    r2 = run_rows("fwd", a_q, a_s, b_q, b_s, [0, 256], 256, 512, mxa.MX_OUT_F32)
    assert np.array_equal(r1, r2)


def test_bf16_epilogue_is_rne_of_fp32_accumulator():
    """The bf16 output of a GEMM is the round-to-nearest-even of the fp32
    output of the same call (same accumulation), element for element."""
    g = np.random.default_rng(9)
    sizes = [300, 0, 517, 64]
    ids = workloads.ids_from_sizes(sizes)
    counts, off, dst, src = routing.route(ids, 4)
    a_q, a_s = routing.permute(*mx_rows(g, (sum(sizes), 640), 1.0, 0.01), src)
    b_q, b_s = mx_rows(g, (4 * 384, 640), 0.02, 0.01)
    b_q, b_s = b_q.reshape(4, 384, 640), b_s.reshape(4, 384, 20)
    f32 = run_rows("fwd", a_q, a_s, b_q, b_s, off, 384, 640, mxa.MX_OUT_F32)
    b16 = run_rows("fwd", a_q, a_s, b_q, b_s, off, 384, 640, mxa.MX_OUT_BF16)
    lo, hi = int(off[0]), int(off[-1])
    assert np.array_equal(b16[lo:hi], mx.f64_to_bf16(f32[lo:hi]))
