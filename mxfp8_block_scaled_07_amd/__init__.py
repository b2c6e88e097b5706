"""MI355X (gfx950) MXFP8 Mixture-of-Experts expert path.

Python binding of ``libmxmoe.so`` (declared in ``include/mxmoe.h``).  The
functions named ``mx_*`` mirror the C entry points one to one and only
marshal arguments: torch tensors stand for device buffers (their data
pointers are passed), ``None`` stands for NULL, and the stream defaults to
torch's current stream.  The ``alloc_*``/convenience helpers only allocate
output tensors with torch and then call the same entry points.  Every
computation runs in the HIP kernels; there is no fallback: if the library is
missing or a call fails, an exception is raised.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxmoe.so")

MX_OK, MX_EINVAL, MX_EUNSUPPORTED, MX_EHIP = 0, -1, -2, -3
MX_OUT_BF16, MX_OUT_F32 = 0, 1

_lib = None

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "mx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mx_quantize": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "mx_dequantize": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "mx_permute_workspace_size": (_sz, [_i64, _i32, _i32]),
    "mx_permute": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mx_permute_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mx_ceiling_copy": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "mx_ceiling_tile_pattern": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "mx_ceiling_mfma": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp]),
    "mx_grouped_gemm_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
    "mx_grouped_gemm_dgrad": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
    "mx_grouped_gemm_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
    "mx_swiglu_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mx_swiglu_bwd_quantize": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mx_combine": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _i64, _i32, _vp, _vp]),
    "mx_combine_bwd_quantize": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                               _vp]),
    "mx_route_topk": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "mx_router_bwd": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "mx_bf16_gather": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "mx_bf16_grouped_gemm_fwd": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
    "mx_bf16_grouped_gemm_dgrad": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
    "mx_bf16_grouped_gemm_wgrad": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp]),
}


class MXError(RuntimeError):
    pass


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MXError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, name):
    if rc != MX_OK:
        raise MXError(f"{name}: {lib().mx_status_string(rc).decode()}")


# --- entry points (same names and argument order as include/mxmoe.h) -------
def mx_quantize(x, batch, rows, cols, gather, rows_out, row_q, row_s, col_q, col_s, stream=None):
    _check(lib().mx_quantize(_p(x), batch, rows, cols, _p(gather), rows_out, _p(row_q), _p(row_s), _p(col_q),
                             _p(col_s), _s(stream)), "mx_quantize")


def mx_dequantize(q, s, rows, cols, y, stream=None):
    _check(lib().mx_dequantize(_p(q), _p(s), rows, cols, _p(y), _s(stream)), "mx_dequantize")


def mx_permute_workspace_size(tokens, topk, num_experts):
    return int(lib().mx_permute_workspace_size(tokens, topk, num_experts))


def mx_permute(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out, group_offsets,
               dst_row, src_row, workspace, workspace_bytes, stream=None):
    _check(lib().mx_permute(_p(q), _p(s), tokens, cols, _p(expert_ids), topk, num_experts, capacity_rows, _p(q_out),
                            _p(s_out), _p(group_offsets), _p(dst_row), _p(src_row), _p(workspace), workspace_bytes,
                            _s(stream)), "mx_permute")


def mx_permute_noalloc(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out,
                       group_offsets, dst_row, src_row, stream=None):
    _check(lib().mx_permute_noalloc(_p(q), _p(s), tokens, cols, _p(expert_ids), topk, num_experts, capacity_rows,
                                    _p(q_out), _p(s_out), _p(group_offsets), _p(dst_row), _p(src_row), _s(stream)),
           "mx_permute_noalloc")


def mx_ceiling_copy(src, dst, nbytes, stream=None):
    _check(lib().mx_ceiling_copy(_p(src), _p(dst), nbytes, _s(stream)), "mx_ceiling_copy")


def mx_ceiling_tile_pattern(x, row_out, col_out, rows, cols, stream=None):
    _check(lib().mx_ceiling_tile_pattern(_p(x), _p(row_out), _p(col_out), rows, cols, _s(stream)),
           "mx_ceiling_tile_pattern")


def mx_ceiling_mfma(out, workgroups, iters, random_operands=True, stream=None):
    _check(lib().mx_ceiling_mfma(_p(out), workgroups, iters, int(bool(random_operands)), _s(stream)),
           "mx_ceiling_mfma")


def mx_grouped_gemm_fwd(a_q, a_s, b_q, b_s, group_offsets, num_groups, m_cap, n, k, out, out_dtype, stream=None):
    _check(lib().mx_grouped_gemm_fwd(_p(a_q), _p(a_s), _p(b_q), _p(b_s), _p(group_offsets), num_groups, m_cap, n, k,
                                     _p(out), out_dtype, _s(stream)), "mx_grouped_gemm_fwd")


def mx_grouped_gemm_dgrad(dy_q, dy_s, wt_q, wt_s, group_offsets, num_groups, m_cap, n_out, k_contract, dx,
                          out_dtype, stream=None):
    _check(lib().mx_grouped_gemm_dgrad(_p(dy_q), _p(dy_s), _p(wt_q), _p(wt_s), _p(group_offsets), num_groups, m_cap,
                                       n_out, k_contract, _p(dx), out_dtype, _s(stream)), "mx_grouped_gemm_dgrad")


def mx_grouped_gemm_wgrad(dyt_q, dyt_s, xt_q, xt_s, group_offsets, num_groups, m_cap, n, k, dw, out_dtype,
                          stream=None):
    _check(lib().mx_grouped_gemm_wgrad(_p(dyt_q), _p(dyt_s), _p(xt_q), _p(xt_s), _p(group_offsets), num_groups, m_cap,
                                       n, k, _p(dw), out_dtype, _s(stream)), "mx_grouped_gemm_wgrad")


def mx_swiglu_quantize(h, rows, F, a, row_q, row_s, col_q, col_s, stream=None):
    _check(lib().mx_swiglu_quantize(_p(h), rows, F, _p(a), _p(row_q), _p(row_s), _p(col_q), _p(col_s), _s(stream)),
           "mx_swiglu_quantize")


def mx_swiglu_bwd_quantize(h, da, rows, F, dh, row_q, row_s, col_q, col_s, stream=None):
    _check(lib().mx_swiglu_bwd_quantize(_p(h), _p(da), rows, F, _p(dh), _p(row_q), _p(row_s), _p(col_q), _p(col_s),
                                        _s(stream)), "mx_swiglu_bwd_quantize")


def mx_combine(y, y_rows, H, dst_row, weights, tokens, topk, out, stream=None):
    _check(lib().mx_combine(_p(y), y_rows, H, _p(dst_row), _p(weights), tokens, topk, _p(out), _s(stream)),
           "mx_combine")


def mx_combine_bwd_quantize(dout, weights, dst_row, src_row, tokens, topk, rows, H, dy, row_q, row_s, col_q, col_s,
                            stream=None):
    _check(lib().mx_combine_bwd_quantize(_p(dout), _p(weights), _p(dst_row), _p(src_row), tokens, topk, rows, H,
                                         _p(dy), _p(row_q), _p(row_s), _p(col_q), _p(col_s), _s(stream)),
           "mx_combine_bwd_quantize")


def mx_route_topk(logits, tokens, num_experts, topk, expert_ids, weights, stream=None):
    _check(lib().mx_route_topk(_p(logits), tokens, num_experts, topk, _p(expert_ids), _p(weights), _s(stream)),
           "mx_route_topk")


def mx_router_bwd(dout, y, y_rows, H, dst_row, expert_ids, weights, tokens, num_experts, topk, dw, dlogits,
                  stream=None):
    _check(lib().mx_router_bwd(_p(dout), _p(y), y_rows, H, _p(dst_row), _p(expert_ids), _p(weights), tokens,
                               num_experts, topk, _p(dw), _p(dlogits), _s(stream)), "mx_router_bwd")


def mx_bf16_gather(x, batch, rows, cols, gather, rows_out, out_rows, out_cols, stream=None):
    _check(lib().mx_bf16_gather(_p(x), batch, rows, cols, _p(gather), rows_out, _p(out_rows), _p(out_cols),
                                _s(stream)), "mx_bf16_gather")


def mx_bf16_grouped_gemm_fwd(a, b, group_offsets, num_groups, m_cap, n, k, out, out_dtype, stream=None):
    _check(lib().mx_bf16_grouped_gemm_fwd(_p(a), _p(b), _p(group_offsets), num_groups, m_cap, n, k, _p(out),
                                          out_dtype, _s(stream)), "mx_bf16_grouped_gemm_fwd")


def mx_bf16_grouped_gemm_dgrad(dy, wt, group_offsets, num_groups, m_cap, n_out, k_contract, dx, out_dtype,
                               stream=None):
    _check(lib().mx_bf16_grouped_gemm_dgrad(_p(dy), _p(wt), _p(group_offsets), num_groups, m_cap, n_out, k_contract,
                                            _p(dx), out_dtype, _s(stream)), "mx_bf16_grouped_gemm_dgrad")


def mx_bf16_grouped_gemm_wgrad(dyt, xt, group_offsets, num_groups, m_cap, n, k, dw, out_dtype, stream=None):
    _check(lib().mx_bf16_grouped_gemm_wgrad(_p(dyt), _p(xt), _p(group_offsets), num_groups, m_cap, n, k, _p(dw),
                                            out_dtype, _s(stream)), "mx_bf16_grouped_gemm_wgrad")


# --- allocating helpers ----------------------------------------------------
def scale_shape(rows, cols):
    """Shape of the scale bytes of an MX tensor with ``rows`` rows (batch
    entries stacked) and ``cols`` columns, in the kernels' panel layout:
    (ceil(cols / 128), rows, 4) -- panel p, row r holds the scale bytes of
    blocks 4p..4p+3 of that row; pad bytes past the last block are zero."""
    return ((cols + 127) // 128, rows, 4)


def quantize(x, rowwise=True, colwise=False, rows_out=None, gather=None, stream=None):
    """x: bf16 (or int16 bit) tensor [rows, cols] or [batch, rows, cols] on the GPU.
    Returns (row_q, row_s, col_q, col_s); unrequested outputs are None."""
    import torch
    if x.dim() == 2:
        batch, rows, cols = 1, x.shape[0], x.shape[1]
    else:
        batch, rows, cols = x.shape
    rows_out = rows if rows_out is None else rows_out
    dev = x.device
    shp = (rows_out, cols) if x.dim() == 2 else (batch, rows_out, cols)
    row_q = torch.empty(shp, dtype=torch.uint8, device=dev) if rowwise else None
    row_s = torch.empty(scale_shape(batch * rows_out, cols), dtype=torch.uint8, device=dev) if rowwise else None
    cshp = (cols, rows_out) if x.dim() == 2 else (batch, cols, rows_out)
    col_q = torch.empty(cshp, dtype=torch.uint8, device=dev) if colwise else None
    col_s = torch.empty(scale_shape(batch * cols, rows_out), dtype=torch.uint8, device=dev) if colwise else None
    mx_quantize(x, batch, rows, cols, gather, rows_out, row_q, row_s, col_q, col_s, stream)
    return row_q, row_s, col_q, col_s


def dequantize(q, s, stream=None):
    """q: codes [..., cols] (leading dims stacked as rows), s: panel-layout scales."""
    import torch
    y = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    mx_dequantize(q, s, q.numel() // q.shape[-1], q.shape[-1], y, stream)
    return y


def permute(q, s, expert_ids, num_experts, capacity_rows=None, stream=None):
    """Returns (q_out, s_out, group_offsets, dst_row, src_row); q/s may be None
    (metadata only)."""
    import torch
    tokens, topk = expert_ids.shape
    dev = expert_ids.device
    cap = -(-(tokens * topk + 31 * num_experts) // 32) * 32 if capacity_rows is None else capacity_rows
    cols = q.shape[1] if q is not None else 0
    q_out = torch.empty((cap, cols), dtype=torch.uint8, device=dev) if q is not None else None
    s_out = torch.empty(scale_shape(cap, cols), dtype=torch.uint8, device=dev) if q is not None else None
    off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    dst = torch.empty(tokens * topk, dtype=torch.int32, device=dev)
    src = torch.empty(cap, dtype=torch.int32, device=dev)
    wsb = mx_permute_workspace_size(tokens, topk, num_experts)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    mx_permute(q, s, tokens, cols, expert_ids, topk, num_experts, cap, q_out, s_out, off, dst, src, ws, wsb, stream)
    return q_out, s_out, off, dst, src


def _mx_pair(rows, cols, dev, want):
    import torch
    if not want:
        return None, None
    return (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
            torch.empty(scale_shape(rows, cols), dtype=torch.uint8, device=dev))


def swiglu_quantize(h, rowwise=True, colwise=True, want_bf16=False, stream=None):
    """h: bf16 [rows, 2F].  Returns (a_bf16, row_q, row_s, col_q, col_s)."""
    import torch
    rows, F = h.shape[0], h.shape[1] // 2
    a = torch.empty((rows, F), dtype=torch.bfloat16, device=h.device) if want_bf16 else None
    rq, rs = _mx_pair(rows, F, h.device, rowwise)
    cq, cs = _mx_pair(F, rows, h.device, colwise)
    if rows:   # an empty input has nothing to compute (its tensors have no storage)
        mx_swiglu_quantize(h, rows, F, a, rq, rs, cq, cs, stream)
    return a, rq, rs, cq, cs


def swiglu_bwd_quantize(h, da, rowwise=True, colwise=True, want_bf16=False, stream=None):
    """h: bf16 [rows, 2F], da: bf16 [rows, F].  Returns (dh_bf16, row_q, row_s, col_q, col_s)."""
    import torch
    rows, F = h.shape[0], h.shape[1] // 2
    dh = torch.empty((rows, 2 * F), dtype=torch.bfloat16, device=h.device) if want_bf16 else None
    rq, rs = _mx_pair(rows, 2 * F, h.device, rowwise)
    cq, cs = _mx_pair(2 * F, rows, h.device, colwise)
    if rows:
        mx_swiglu_bwd_quantize(h, da, rows, F, dh, rq, rs, cq, cs, stream)
    return dh, rq, rs, cq, cs


def combine(y, dst_row, weights, tokens, topk, stream=None):
    """y: bf16 [rows, H] permuted rows; weights fp32 [tokens, topk] or None.  Returns bf16 [tokens, H]."""
    import torch
    out = torch.empty((tokens, y.shape[1]), dtype=torch.bfloat16, device=y.device)
    if tokens:
        mx_combine(y, y.shape[0], y.shape[1], dst_row, weights, tokens, topk, out, stream)
    return out


def combine_bwd_quantize(dout, weights, dst_row, src_row, topk, rows, rowwise=True, colwise=True, want_bf16=False,
                         stream=None):
    """dout: bf16 [tokens, H].  Returns (dy_bf16, row_q, row_s, col_q, col_s) of the permuted gradient [rows, H]."""
    import torch
    tokens, H = dout.shape
    dy = torch.empty((rows, H), dtype=torch.bfloat16, device=dout.device) if want_bf16 else None
    rq, rs = _mx_pair(rows, H, dout.device, rowwise)
    cq, cs = _mx_pair(H, rows, dout.device, colwise)
    if rows:
        mx_combine_bwd_quantize(dout if tokens else None, weights if tokens else None, dst_row if tokens else None,
                                src_row, tokens, topk, rows, H, dy, rq, rs, cq, cs, stream)
    return dy, rq, rs, cq, cs


def route_topk(logits, topk, stream=None):
    """logits: fp32 [tokens, E].  Returns (expert_ids int32 [tokens, topk], weights fp32 [tokens, topk])."""
    import torch
    T, E = logits.shape
    ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    if T:
        mx_route_topk(logits, T, E, topk, ids, w, stream)
    return ids, w


def router_bwd(dout, y, dst_row, expert_ids, weights, num_experts, stream=None):
    """Returns (dw fp32 [tokens, topk], dlogits fp32 [tokens, num_experts])."""
    import torch
    T, topk = weights.shape
    dw = torch.empty((T, topk), dtype=torch.float32, device=dout.device)
    dl = torch.empty((T, num_experts), dtype=torch.float32, device=dout.device)
    if T:
        mx_router_bwd(dout, y, y.shape[0], y.shape[1], dst_row, expert_ids, weights, T, num_experts, topk, dw, dl,
                      stream)
    return dw, dl
