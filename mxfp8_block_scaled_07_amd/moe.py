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

from . import (MX_OUT_BF16, MX_OUT_F32, mx_grouped_gemm_dgrad, mx_grouped_gemm_fwd, mx_grouped_gemm_wgrad,
               mx_permute, mx_permute_workspace_size, mx_quantize, scale_shape)

STAGES = ("quant_x", "permute", "quant_w", "gemm_fwd", "quant_dy", "gemm_dgrad", "quant_xt", "gemm_wgrad")


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
    elif name == "gemm_wgrad":
        mx_grouped_gemm_wgrad(b.dytq, b.dyts, b.xtq, b.xts, b.off, E, cap, N, K, b.dw, od, stream)
    else:
        raise ValueError(name)


def expert_step(b, x, w, dy, expert_ids, stream=None):
    """One forward + backward pass of the expert computation."""
    for name in STAGES:
        run_stage(name, b, x, w, dy, expert_ids, stream)


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
        },
    }
