"""The MXFP8 MoE expert computation, forward plus backward, as one call chain
over the C ABI (every step runs in the HIP kernels; torch only provides the
device buffers and the stream).

Steps (the expert part of the MXFP8 MoE layer of the MXFP8 MoE digest,
Overview; pytorch/ao PR #3203 "Next steps": quantize once, shuffle tokens in
MXFP8, grouped GEMM on pre-quantized tensors):

  1. X rowwise quantize                      mx_quantize
  2. route + permute X in MXFP8              mx_permute
  3. W rowwise + columnwise quantize         mx_quantize (batch = experts)
  4. Y = X_perm W_e^T                        mx_grouped_gemm_fwd
  5. dY rowwise + columnwise quantize        mx_quantize
  6. dX_perm = dY W_e                        mx_grouped_gemm_dgrad
  7. X columnwise quantize in permuted order mx_quantize (gather = src_row)
  8. dW_e = dY_e^T X_e                       mx_grouped_gemm_wgrad

dY arrives in the padded permuted layout with zero pad rows (the layout the
combine backward writes); ``zero_pad_rows`` prepares such a tensor.
"""

import torch

from . import (MX_OUT_BF16, MX_OUT_F32, mx_bf16_gather, mx_bf16_grouped_gemm_dgrad, mx_bf16_grouped_gemm_fwd,
               mx_bf16_grouped_gemm_wgrad, mx_combine, mx_combine_bwd_quantize, mx_grouped_gemm_dgrad,
               mx_grouped_gemm_fwd, mx_grouped_gemm_wgrad, mx_permute, mx_permute_workspace_size, mx_quantize,
               mx_route_topk, mx_router_bwd, mx_swiglu_bwd_quantize, mx_swiglu_quantize, scale_shape)

STAGES = ("quant_x", "permute", "quant_w", "gemm_fwd", "quant_dy", "gemm_dgrad", "quant_xt", "gemm_wgrad")

# The same computation with the quantize fused into the permute (PR #3203
# "Next steps" lists fusing the cast and the token shuffle): routing metadata
# only, then one gathered pass over the bf16 tokens that writes the permuted
# rowwise MX (GEMM fwd operand) and the columnwise MX in permuted order (wgrad
# operand).  Rowwise quantization is per row, so quantize-then-permute and
# permute-then-quantize give the same bytes; the MXFP8 permute stays the step
# of choice when the token shuffle is a transfer between devices.
FUSED_STAGES = ("route", "quant_xperm", "quant_w", "gemm_fwd", "quant_dy", "gemm_dgrad", "gemm_wgrad")


class ExpertBuffers:
    """Device buffers for one (T, K, N, E, topk) problem, allocated once."""

    def __init__(self, T, K, N, E, topk, device="cuda:0", out_dtype=MX_OUT_BF16):
        self.T, self.K, self.N, self.E, self.topk = T, K, N, E, topk
        self.cap = -(-(T * topk + 31 * E) // 32) * 32  # worst case, rounded to whole 32-row blocks
        self.out_dtype = out_dtype
        u8, i32 = torch.uint8, torch.int32
        od = torch.bfloat16 if out_dtype == MX_OUT_BF16 else torch.float32
        cap = self.cap
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        sc = lambda r, c: e(*scale_shape(r, c))  # noqa: E731  panel-layout scales
        self.xq, self.xs = e(T, K), sc(T, K)
        self.xpq, self.xps = e(cap, K), sc(cap, K)
        self.off, self.dst, self.src = e(E + 1, dt=i32), e(T * topk, dt=i32), e(cap, dt=i32)
        self.wsb = mx_permute_workspace_size(T, topk, E)
        self.ws = e(max(self.wsb, 4))
        self.wq, self.wsc = e(E, N, K), sc(E * N, K)
        self.wtq, self.wtsc = e(E, K, N), sc(E * K, N)
        self.dyq, self.dys = e(cap, N), sc(cap, N)
        self.dytq, self.dyts = e(N, cap), sc(N, cap)
        self.xtq, self.xts = e(K, cap), sc(K, cap)
        self.y = e(cap, N, dt=od)
        self.dx = e(cap, K, dt=od)
        self.dw = e(E, N, K, dt=od)


def run_stage(name, b, x, w, dy, expert_ids, stream=None):
    """Launch one named stage on ``stream`` (default: torch's current stream)."""
    T, K, N, E, topk, cap, od = b.T, b.K, b.N, b.E, b.topk, b.cap, b.out_dtype
    if name == "quant_x":
        mx_quantize(x, 1, T, K, None, T, b.xq, b.xs, None, None, stream)
    elif name == "permute":
        mx_permute(b.xq, b.xs, T, K, expert_ids, topk, E, cap, b.xpq, b.xps, b.off, b.dst, b.src, b.ws, b.wsb, stream)
    elif name == "quant_w":
        mx_quantize(w, E, N, K, None, N, b.wq, b.wsc, b.wtq, b.wtsc, stream)
    elif name == "gemm_fwd":
        mx_grouped_gemm_fwd(b.xpq, b.xps, b.wq, b.wsc, b.off, E, cap, N, K, b.y, od, stream)
    elif name == "quant_dy":
        mx_quantize(dy, 1, cap, N, None, cap, b.dyq, b.dys, b.dytq, b.dyts, stream)
    elif name == "gemm_dgrad":
        mx_grouped_gemm_dgrad(b.dyq, b.dys, b.wtq, b.wtsc, b.off, E, cap, K, N, b.dx, od, stream)
    elif name == "quant_xt":
        mx_quantize(x, 1, T, K, b.src, cap, None, None, b.xtq, b.xts, stream)
    elif name == "route":
        mx_permute(None, None, T, K, expert_ids, topk, E, cap, None, None, b.off, b.dst, b.src, b.ws, b.wsb, stream)
    elif name == "quant_xperm":
        mx_quantize(x, 1, T, K, b.src, cap, b.xpq, b.xps, b.xtq, b.xts, stream)
    elif name == "gemm_wgrad":
        mx_grouped_gemm_wgrad(b.dytq, b.dyts, b.xtq, b.xts, b.off, E, cap, N, K, b.dw, od, stream)
    else:
        raise ValueError(name)


def expert_step(b, x, w, dy, expert_ids, stream=None):
    """One forward + backward pass of the expert computation."""
    for name in STAGES:
        run_stage(name, b, x, w, dy, expert_ids, stream)


def fused_expert_step(b, x, w, dy, expert_ids, stream=None):
    """The same pass with the quantize fused into the permute (FUSED_STAGES);
    leaves b.xq / b.xs (the unpermuted rowwise MX) unwritten."""
    for name in FUSED_STAGES:
        run_stage(name, b, x, w, dy, expert_ids, stream)


# The BF16 baseline of the same step (the digest's Overview compares the
# MXFP8 MoE layer with a BF16 one): the same routing, the tokens gathered
# into expert order in bf16, the operands the GEMMs read along the other axis
# transposed in bf16 (the counterpart of the columnwise quantizes), and the
# three grouped GEMMs on bf16 operands.
BF16_STAGES = ("route", "permute_bf16", "transpose_w", "gemm_fwd", "transpose_dy", "gemm_dgrad", "transpose_xt",
               "gemm_wgrad")


class Bf16Buffers:
    """Device buffers of the BF16 step for one (T, K, N, E, topk) problem."""

    def __init__(self, T, K, N, E, topk, device="cuda:0", out_dtype=MX_OUT_BF16):
        self.T, self.K, self.N, self.E, self.topk = T, K, N, E, topk
        self.cap = -(-(T * topk + 31 * E) // 32) * 32
        self.out_dtype = out_dtype
        bf, i32 = torch.bfloat16, torch.int32
        od = torch.bfloat16 if out_dtype == MX_OUT_BF16 else torch.float32
        cap = self.cap
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        self.off, self.dst, self.src = e(E + 1, dt=i32), e(T * topk, dt=i32), e(cap, dt=i32)
        self.wsb = mx_permute_workspace_size(T, topk, E)
        self.ws = e(max(self.wsb, 4), dt=torch.uint8)
        self.xp = e(cap, K)
        self.wt = e(E, K, N)
        self.dyt = e(N, cap)
        self.xt = e(K, cap)
        self.y = e(cap, N, dt=od)
        self.dx = e(cap, K, dt=od)
        self.dw = e(E, N, K, dt=od)


def run_bf16_stage(name, b, x, w, dy, expert_ids, stream=None):
    """Launch one named stage of the BF16 step on ``stream``."""
    T, K, N, E, topk, cap, od = b.T, b.K, b.N, b.E, b.topk, b.cap, b.out_dtype
    if name == "route":
        mx_permute(None, None, T, K, expert_ids, topk, E, cap, None, None, b.off, b.dst, b.src, b.ws, b.wsb, stream)
    elif name == "permute_bf16":
        mx_bf16_gather(x, 1, T, K, b.src, cap, b.xp, None, stream)
    elif name == "transpose_w":
        mx_bf16_gather(w, E, N, K, None, N, None, b.wt, stream)
    elif name == "gemm_fwd":
        mx_bf16_grouped_gemm_fwd(b.xp, w, b.off, E, cap, N, K, b.y, od, stream)
    elif name == "transpose_dy":
        mx_bf16_gather(dy, 1, cap, N, None, cap, None, b.dyt, stream)
    elif name == "gemm_dgrad":
        mx_bf16_grouped_gemm_dgrad(dy, b.wt, b.off, E, cap, K, N, b.dx, od, stream)
    elif name == "transpose_xt":
        mx_bf16_gather(x, 1, T, K, b.src, cap, None, b.xt, stream)
    elif name == "gemm_wgrad":
        mx_bf16_grouped_gemm_wgrad(b.dyt, b.xt, b.off, E, cap, N, K, b.dw, od, stream)
    else:
        raise ValueError(name)


def bf16_expert_step(b, x, w, dy, expert_ids, stream=None):
    """One forward + backward pass of the BF16 baseline step."""
    for name in BF16_STAGES:
        run_bf16_stage(name, b, x, w, dy, expert_ids, stream)


def bf16_work(T, K, N, E, topk, m_real=None):
    """Bytes of the BF16 step's layout stages and of its GEMM operands (bf16
    operands, bf16 outputs); the GEMM FLOPs are those of algorithmic_work."""
    M = T * topk if m_real is None else m_real
    cap = -(-(T * topk + 31 * E) // 32) * 32
    return {
        "gemm_operand_bytes": {"gemm_fwd": (M * K + E * N * K) * 2 + M * N * 2,
                               "gemm_dgrad": (M * N + E * K * N) * 2 + M * K * 2,
                               "gemm_wgrad": (N * M + K * M) * 2 + E * N * K * 2},
        "bytes": {
            "route": 4 * (T * topk * 2 + cap),
            "permute_bf16": M * K * 2 + cap * K * 2 + 4 * cap,
            "transpose_w": E * N * K * 4,
            "transpose_dy": cap * N * 4,
            "transpose_xt": M * K * 2 + cap * K * 2 + 4 * cap,
        },
    }


def capture(fn, warm=2):
    """Capture one call of ``fn`` -- a step whose calls launch on torch's
    current stream and allocate nothing -- into a HIP graph
    (torch.cuda.CUDAGraph); ``graph.replay()`` then relaunches the whole step
    without host launch overhead.  ``fn`` runs ``warm`` times on a side
    stream first.  The library's kernels write every output they own on each
    call, so a replay reproduces the eager step bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warm):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def zero_pad_rows(dy_full, src_row):
    """dY in the padded permuted layout: rows whose src_row is -1 (pad rows
    and rows past the last group) set to zero (test/bench input preparation)."""
    dy = dy_full.clone()
    dy[src_row < 0] = 0
    return dy


def algorithmic_work(T, K, N, E, topk, m_real=None):
    """FLOPs of the three GEMMs (real rows only) and bytes of every stage."""
    M = T * topk if m_real is None else m_real
    cap = -(-(T * topk + 31 * E) // 32) * 32
    gemm = 2.0 * M * N * K
    # operand and output bytes each GEMM must move at least once: A and B codes
    # plus scales (1 + 1/32 B per element) and a bf16 output
    fwd_b = (M * K + E * N * K) * (1 + 1 / 32) + M * N * 2
    dgrad_b = (M * N + E * K * N) * (1 + 1 / 32) + M * K * 2
    wgrad_b = (N * M + K * M) * (1 + 1 / 32) + E * N * K * 2
    row_b = lambda r, c: r * c * (2 + 1 + 1 / 32)              # noqa: E731  bf16 in, codes + scales out
    rowcol_b = lambda r, c: r * c * (2 + 2 * (1 + 1 / 32))     # noqa: E731
    return {
        "gemm_flops": {"gemm_fwd": gemm, "gemm_dgrad": gemm, "gemm_wgrad": gemm},
        "gemm_operand_bytes": {"gemm_fwd": fwd_b, "gemm_dgrad": dgrad_b, "gemm_wgrad": wgrad_b},
        "bytes": {
            "quant_x": row_b(T, K),
            "permute": K * (1 + 1 / 32) * (T + cap) + 4 * (T * topk * 2 + cap),
            "quant_w": rowcol_b(E * N, K),
            "quant_dy": rowcol_b(cap, N),
            "quant_xt": M * K * 2 + cap * K * (1 + 1 / 32) + 4 * cap,
            "route": 4 * (T * topk * 2 + cap),
            "quant_xperm": M * K * 2 + 2 * cap * K * (1 + 1 / 32) + 4 * cap,
        },
    }


# ---------------------------------------------------------------------------
# The SwiGLU expert FFN layer: router -> permute -> gate/up GEMM -> SwiGLU ->
# down GEMM -> weighted combine, forward and backward (down to the router
# logits), every operand of every GEMM in MXFP8.  W1 [E, 2F, H] holds the gate rows [0, F) and the up rows [F, 2F)
# of each expert; W2 [E, H, F].
# ---------------------------------------------------------------------------
LAYER_STAGES = ("router", "quant_x", "permute", "quant_w1", "gemm1_fwd", "swiglu", "quant_w2", "gemm2_fwd",
                "combine", "combine_bwd", "router_bwd", "gemm2_dgrad", "gemm2_wgrad", "swiglu_bwd", "gemm1_dgrad",
                "quant_xt", "gemm1_wgrad", "unpermute_dx")
# the same layer with the quantize fused into the permute (as FUSED_STAGES)
LAYER_FUSED_STAGES = ("router", "route", "quant_xperm", "quant_w1", "gemm1_fwd", "swiglu", "quant_w2", "gemm2_fwd",
                      "combine", "combine_bwd", "router_bwd", "gemm2_dgrad", "gemm2_wgrad", "swiglu_bwd",
                      "gemm1_dgrad", "gemm1_wgrad", "unpermute_dx")


class LayerBuffers:
    """Device buffers of one SwiGLU expert FFN layer (T tokens, hidden H,
    expert ffn F, E experts, top-k), allocated once.  Buffers that a kernel
    reads over all capacity rows but a grouped GEMM only writes inside the
    groups (h, da) start zeroed, so rows past the last group stay zero."""

    def __init__(self, T, H, F, E, topk, device="cuda:0"):
        self.T, self.H, self.F, self.E, self.topk = T, H, F, E, topk
        self.cap = cap = -(-(T * topk + 31 * E) // 32) * 32
        u8, i32, bf = torch.uint8, torch.int32, torch.bfloat16
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        sc = lambda r, c: e(*scale_shape(r, c))  # noqa: E731
        self.xq, self.xs = e(T, H), sc(T, H)
        self.xpq, self.xps = e(cap, H), sc(cap, H)
        self.ids, self.weights = e(T, topk, dt=i32), e(T, topk, dt=torch.float32)
        self.off, self.dst, self.src = e(E + 1, dt=i32), e(T * topk, dt=i32), e(cap, dt=i32)
        self.wsb = mx_permute_workspace_size(T, topk, E)
        self.ws = e(max(self.wsb, 4))
        self.dweights, self.dlogits = e(T, topk, dt=torch.float32), e(T, E, dt=torch.float32)
        self.w1q, self.w1s = e(E, 2 * F, H), sc(E * 2 * F, H)
        self.w1tq, self.w1ts = e(E, H, 2 * F), sc(E * H, 2 * F)
        self.w2q, self.w2s = e(E, H, F), sc(E * H, F)
        self.w2tq, self.w2ts = e(E, F, H), sc(E * F, H)
        self.h = torch.zeros((cap, 2 * F), dtype=bf, device=device)
        self.aq, self.as_ = e(cap, F), sc(cap, F)
        self.atq, self.ats = e(F, cap), sc(F, cap)
        self.y = e(cap, H, dt=bf)
        self.out = e(T, H, dt=bf)
        self.dyq, self.dys = e(cap, H), sc(cap, H)
        self.dytq, self.dyts = e(H, cap), sc(H, cap)
        self.da = torch.zeros((cap, F), dtype=bf, device=device)
        self.dw2 = e(E, H, F, dt=bf)
        self.dhq, self.dhs = e(cap, 2 * F), sc(cap, 2 * F)
        self.dhtq, self.dhts = e(2 * F, cap), sc(2 * F, cap)
        self.dxp = e(cap, H, dt=bf)
        self.xtq, self.xts = e(H, cap), sc(H, cap)
        self.dw1 = e(E, 2 * F, H, dt=bf)
        self.dx = e(T, H, dt=bf)


def run_layer_stage(name, b, x, w1, w2, logits, dout, stream=None):
    """Launch one named stage of the layer on ``stream`` (default: torch's current stream)."""
    T, H, F, E, k, cap, bf = b.T, b.H, b.F, b.E, b.topk, b.cap, MX_OUT_BF16
    ids, weights = b.ids, b.weights
    if name == "router":
        mx_route_topk(logits, T, E, k, b.ids, b.weights, stream)
    elif name == "quant_x":
        mx_quantize(x, 1, T, H, None, T, b.xq, b.xs, None, None, stream)
    elif name == "permute":
        mx_permute(b.xq, b.xs, T, H, ids, k, E, cap, b.xpq, b.xps, b.off, b.dst, b.src, b.ws, b.wsb, stream)
    elif name == "route":
        mx_permute(None, None, T, H, ids, k, E, cap, None, None, b.off, b.dst, b.src, b.ws, b.wsb, stream)
    elif name == "quant_xperm":
        mx_quantize(x, 1, T, H, b.src, cap, b.xpq, b.xps, b.xtq, b.xts, stream)
    elif name == "quant_w1":
        mx_quantize(w1, E, 2 * F, H, None, 2 * F, b.w1q, b.w1s, b.w1tq, b.w1ts, stream)
    elif name == "gemm1_fwd":
        mx_grouped_gemm_fwd(b.xpq, b.xps, b.w1q, b.w1s, b.off, E, cap, 2 * F, H, b.h, bf, stream)
    elif name == "swiglu":
        mx_swiglu_quantize(b.h, cap, F, None, b.aq, b.as_, b.atq, b.ats, stream)
    elif name == "quant_w2":
        mx_quantize(w2, E, H, F, None, H, b.w2q, b.w2s, b.w2tq, b.w2ts, stream)
    elif name == "gemm2_fwd":
        mx_grouped_gemm_fwd(b.aq, b.as_, b.w2q, b.w2s, b.off, E, cap, H, F, b.y, bf, stream)
    elif name == "combine":
        mx_combine(b.y, cap, H, b.dst, weights, T, k, b.out, stream)
    elif name == "combine_bwd":
        mx_combine_bwd_quantize(dout, weights, b.dst, b.src, T, k, cap, H, None, b.dyq, b.dys, b.dytq, b.dyts,
                                stream)
    elif name == "router_bwd":
        mx_router_bwd(dout, b.y, cap, H, b.dst, b.ids, b.weights, T, E, k, b.dweights, b.dlogits, stream)
    elif name == "gemm2_dgrad":
        mx_grouped_gemm_dgrad(b.dyq, b.dys, b.w2tq, b.w2ts, b.off, E, cap, F, H, b.da, bf, stream)
    elif name == "gemm2_wgrad":
        mx_grouped_gemm_wgrad(b.dytq, b.dyts, b.atq, b.ats, b.off, E, cap, H, F, b.dw2, bf, stream)
    elif name == "swiglu_bwd":
        mx_swiglu_bwd_quantize(b.h, b.da, cap, F, None, b.dhq, b.dhs, b.dhtq, b.dhts, stream)
    elif name == "gemm1_dgrad":
        mx_grouped_gemm_dgrad(b.dhq, b.dhs, b.w1tq, b.w1ts, b.off, E, cap, H, 2 * F, b.dxp, bf, stream)
    elif name == "quant_xt":
        mx_quantize(x, 1, T, H, b.src, cap, None, None, b.xtq, b.xts, stream)
    elif name == "gemm1_wgrad":
        mx_grouped_gemm_wgrad(b.dhtq, b.dhts, b.xtq, b.xts, b.off, E, cap, 2 * F, H, b.dw1, bf, stream)
    elif name == "unpermute_dx":
        mx_combine(b.dxp, cap, H, b.dst, None, T, k, b.dx, stream)
    else:
        raise ValueError(name)


def layer_step(b, x, w1, w2, logits, dout, stream=None):
    """One forward + backward pass of the SwiGLU expert FFN layer."""
    for name in LAYER_STAGES:
        run_layer_stage(name, b, x, w1, w2, logits, dout, stream)


def fused_layer_step(b, x, w1, w2, logits, dout, stream=None):
    """The same pass with the quantize fused into the permute
    (LAYER_FUSED_STAGES); leaves b.xq / b.xs unwritten."""
    for name in LAYER_FUSED_STAGES:
        run_layer_stage(name, b, x, w1, w2, logits, dout, stream)


def layer_work(T, H, F, E, topk):
    """FLOPs of the six GEMMs (real routed rows only) and the algorithmic
    bytes of every other stage (each tensor read or written once)."""
    M = T * topk
    cap = -(-(T * topk + 31 * E) // 32) * 32
    mx = 1 + 1 / 32
    g1 = 2.0 * M * 2 * F * H
    g2 = 2.0 * M * H * F
    return {
        "gemm_flops": {"gemm1_fwd": g1, "gemm2_fwd": g2, "gemm2_dgrad": g2, "gemm2_wgrad": g2,
                       "gemm1_dgrad": g1, "gemm1_wgrad": g1},
        # MX operands (codes + scales) read once and the bf16 output written once
        "gemm_operand_bytes": {
            "gemm1_fwd": (M * H + E * 2 * F * H) * mx + M * 2 * F * 2,
            "gemm2_fwd": (M * F + E * H * F) * mx + M * H * 2,
            "gemm2_dgrad": (M * H + E * F * H) * mx + M * F * 2,
            "gemm2_wgrad": (H * M + F * M) * mx + E * H * F * 2,
            "gemm1_dgrad": (M * 2 * F + E * H * 2 * F) * mx + M * H * 2,
            "gemm1_wgrad": (2 * F * M + H * M) * mx + E * 2 * F * H * 2,
        },
        "bytes": {
            "router": T * E * 4 + M * 8,                            # logits in, ids + weights out
            "router_bwd": T * H * (2 * topk + 2) + M * 16 + T * E * 4,   # dOut and k rows of Y in, dw + dlogits out
            "quant_x": T * H * (2 + mx),
            "permute": H * mx * (T + cap) + 4 * (M * 2 + cap),
            "quant_w1": E * 2 * F * H * (2 + 2 * mx),
            "swiglu": cap * F * (4 + 2 * mx),                       # read g, u; write A row + col MX
            "quant_w2": E * H * F * (2 + 2 * mx),
            "combine": T * H * (2 * topk + 2) + M * 8,              # k rows in, one row out, ids + weights
            "combine_bwd": T * H * 2 + cap * H * 2 * mx + M * 8 + cap * 4,
            "swiglu_bwd": cap * F * 6 + cap * 2 * F * 2 * mx,       # read g, u, dA; write dH row + col MX
            "quant_xt": M * H * 2 + cap * H * mx + 4 * cap,
            "route": 4 * (M * 2 + cap),
            "quant_xperm": M * H * 2 + 2 * cap * H * mx + 4 * cap,
            "unpermute_dx": T * H * (2 * topk + 2) + M * 4,
        },
    }
