"""The C-ABI library loads without a GPU, exports every function that
include/mxmoe.h declares, and rejects invalid host-side arguments with the
documented status codes before touching the GPU."""

import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_07_amd as mxa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mxmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mxa.LIB_PATH):
        from mxfp8_block_scaled_07_amd import _build
        _build.build()
    return mxa.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"mx_quantize", "mx_dequantize", "mx_permute", "mx_permute_workspace_size",
                          "mx_grouped_gemm_fwd", "mx_grouped_gemm_dgrad", "mx_grouped_gemm_wgrad",
                          "mx_status_string", "mx_swiglu_quantize", "mx_swiglu_bwd_quantize", "mx_combine",
                          "mx_combine_bwd_quantize", "mx_route_topk", "mx_router_bwd", "mx_bf16_gather",
                          "mx_bf16_grouped_gemm_fwd", "mx_bf16_grouped_gemm_dgrad", "mx_bf16_grouped_gemm_wgrad"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.mx_status_string(0) == b"MX_OK"
    assert lib.mx_status_string(-1).startswith(b"MX_EINVAL")
    assert lib.mx_status_string(-3).startswith(b"MX_EHIP")


P = ctypes.c_void_p(16)  # a non-null dummy pointer: never dereferenced on these paths


def test_quantize_validation(lib):
    q = lib.mx_quantize
    assert q(None, 1, 32, 32, None, 32, P, P, None, None, None) == mxa.MX_EINVAL          # x null
    assert q(P, 1, 32, 48, None, 32, P, P, None, None, None) == mxa.MX_EINVAL             # cols % 32
    assert q(P, 1, 32, 32, None, 32, None, None, None, None, None) == mxa.MX_EINVAL       # no output
    assert q(P, 1, 32, 32, None, 32, P, None, None, None, None) == mxa.MX_EINVAL          # half a pair
    assert q(P, 1, 32, 32, None, 40, None, None, P, P, None) == mxa.MX_EINVAL             # colwise rows_out % 32
    assert q(P, 2, 32, 32, P, 32, P, P, None, None, None) == mxa.MX_EINVAL                # gather with batch
    assert q(P, 1, 32, 32, None, 0, P, P, None, None, None) == mxa.MX_OK                  # empty: no launch


def test_dequantize_validation(lib):
    d = lib.mx_dequantize
    assert d(None, P, 4, 32, P, None) == mxa.MX_EINVAL
    assert d(P, P, 4, 33, P, None) == mxa.MX_EINVAL
    assert d(P, P, 0, 32, P, None) == mxa.MX_OK


def test_permute_validation(lib):
    ws = lib.mx_permute_workspace_size(100, 2, 4)
    assert ws >= 2 * 4 * 4
    p = lib.mx_permute
    # capacity below tokens*topk + 31*E
    assert p(P, P, 100, 64, P, 2, 4, 200 + 31 * 4 - 1, P, P, P, P, P, P, ws, None) == mxa.MX_EINVAL
    # workspace too small
    assert p(P, P, 100, 64, P, 2, 4, 400, P, P, P, P, P, P, ws - 1, None) == mxa.MX_EINVAL
    # copy requested with a missing output
    assert p(P, P, 100, 64, P, 2, 4, 400, None, P, P, P, P, P, ws, None) == mxa.MX_EINVAL
    assert p(None, None, 100, 0, P, 0, 4, 400, None, None, P, P, P, P, ws, None) == mxa.MX_EINVAL   # topk 0
    # more experts than the routing kernels hold in LDS: a valid request this library does not implement
    E = 16385
    wsb = lib.mx_permute_workspace_size(100, 2, E)
    assert p(None, None, 100, 0, P, 2, E, 200 + 31 * E, None, None, P, P, P, P, wsb, None) == mxa.MX_EUNSUPPORTED


def test_gemm_validation(lib):
    for fn in (lib.mx_grouped_gemm_fwd, lib.mx_grouped_gemm_dgrad):
        assert fn(P, P, P, P, P, 2, 64, 48, 64, P, 0, None) == mxa.MX_EINVAL   # n % 32
        assert fn(P, P, P, P, P, 2, 64, 64, 40, P, 0, None) == mxa.MX_EINVAL   # k % 32
        assert fn(P, P, P, P, P, 0, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL   # no groups
        assert fn(P, P, P, P, P, 2, 64, 64, 64, P, 7, None) == mxa.MX_EINVAL   # dtype
        assert fn(P, P, None, P, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL
        assert fn(P, P, P, P, P, 2, 0, 64, 64, P, 0, None) == mxa.MX_OK        # no rows: nothing to do
        assert fn(P, P, P, P, P, 5000, 64, 64, 64, P, 0, None) == mxa.MX_EUNSUPPORTED  # too many groups
    w = lib.mx_grouped_gemm_wgrad
    assert w(P, P, P, P, P, 2, 48, 64, 64, P, 0, None) == mxa.MX_EINVAL        # m_cap % 32
    assert w(P, P, P, P, None, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL


Q = ctypes.c_void_p(8)  # 8-byte aligned only: rejected where 16-byte loads or stores need alignment


def test_quantize_alignment(lib):
    q = lib.mx_quantize
    assert q(Q, 1, 32, 32, None, 32, P, P, None, None, None) == mxa.MX_EINVAL             # x not 16-aligned
    assert q(P, 1, 32, 32, None, 32, None, None, Q, P, None) == mxa.MX_EINVAL             # col codes
    assert q(P, 1, 32, 32, None, 32, P, ctypes.c_void_p(18), None, None, None) == mxa.MX_EINVAL   # scales


def test_gemm_alignment(lib):
    """Codes feed 16-byte LDS-direct loads and outputs take 16-byte stores:
    misaligned code or output pointers are rejected (scales need 4 bytes)."""
    for fn in (lib.mx_grouped_gemm_fwd, lib.mx_grouped_gemm_dgrad, lib.mx_grouped_gemm_wgrad):
        assert fn(Q, P, P, P, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL      # a codes
        assert fn(P, P, Q, P, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL      # b codes
        assert fn(P, P, P, P, P, 2, 64, 64, 64, Q, 0, None) == mxa.MX_EINVAL      # output
        assert fn(P, ctypes.c_void_p(18), P, P, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL   # a scales
        assert fn(P, P, P, ctypes.c_void_p(18), P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL   # b scales
    for fn in (lib.mx_bf16_grouped_gemm_fwd, lib.mx_bf16_grouped_gemm_dgrad, lib.mx_bf16_grouped_gemm_wgrad):
        assert fn(P, P, P, 2, 64, 64, 64, Q, 0, None) == mxa.MX_EINVAL            # output


def test_dequantize_alignment(lib):
    d = lib.mx_dequantize
    assert d(Q, P, 4, 32, P, None) == mxa.MX_EINVAL                                # codes
    assert d(P, P, 4, 32, Q, None) == mxa.MX_EINVAL                                # bf16 output
    assert d(P, ctypes.c_void_p(18), 4, 32, P, None) == mxa.MX_EINVAL              # scales


def test_permute_grid_limit_checked_before_any_launch(lib):
    """A copy grid beyond 2^31 - 1 blocks is rejected up front (before the
    routing kernels are enqueued); on a machine without a GPU any launch
    would return MX_EHIP instead."""
    tokens = (1 << 31) - 100
    cap = tokens + 31
    ws = lib.mx_permute_workspace_size(tokens, 1, 1)
    assert ws > 0
    p = lib.mx_permute
    assert p(P, P, tokens, 32, P, 1, 1, cap, P, P, P, P, P, P, ws, None) == mxa.MX_EINVAL


def test_permute_code_alignment(lib):
    ws = lib.mx_permute_workspace_size(100, 2, 4)
    p = lib.mx_permute
    assert p(Q, P, 100, 64, P, 2, 4, 400, P, P, P, P, P, P, ws, None) == mxa.MX_EINVAL   # codes not 16-aligned
    assert p(P, P, 100, 64, P, 2, 4, 400, Q, P, P, P, P, P, ws, None) == mxa.MX_EINVAL


def test_bf16_validation(lib):
    g = lib.mx_bf16_gather
    assert g(None, 1, 64, 64, None, 64, P, None, None) == mxa.MX_EINVAL        # x null
    assert g(P, 1, 64, 64, None, 64, None, None, None) == mxa.MX_EINVAL        # no output
    assert g(P, 1, 64, 48, None, 64, P, None, None) == mxa.MX_EINVAL           # cols % 32
    assert g(P, 1, 64, 64, None, 48, P, None, None) == mxa.MX_EINVAL           # rows_out % 32
    assert g(P, 1, 64, 64, None, 32, P, None, None) == mxa.MX_EINVAL           # rows_out < rows, no gather
    assert g(P, 2, 64, 64, P, 64, P, None, None) == mxa.MX_EINVAL              # gather with batch > 1
    assert g(Q, 1, 64, 64, None, 64, P, None, None) == mxa.MX_EINVAL           # x not 16-aligned
    assert g(P, 1, 0, 64, None, 0, P, None, None) == mxa.MX_OK                 # no rows: nothing to do
    for fn in (lib.mx_bf16_grouped_gemm_fwd, lib.mx_bf16_grouped_gemm_dgrad):
        assert fn(P, P, P, 2, 64, 48, 64, P, 0, None) == mxa.MX_EINVAL          # n % 32
        assert fn(P, P, P, 2, 64, 64, 40, P, 0, None) == mxa.MX_EINVAL          # k % 32
        assert fn(P, P, P, 0, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL          # no groups
        assert fn(P, P, P, 2, 64, 64, 64, P, 7, None) == mxa.MX_EINVAL          # dtype
        assert fn(Q, P, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL          # a not 16-aligned
        assert fn(P, P, None, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL       # offsets null
        assert fn(P, P, P, 2, 0, 64, 64, P, 0, None) == mxa.MX_OK               # no rows
        assert fn(P, P, P, 5000, 64, 64, 64, P, 0, None) == mxa.MX_EUNSUPPORTED  # too many groups
    w = lib.mx_bf16_grouped_gemm_wgrad
    assert w(P, P, P, 2, 48, 64, 64, P, 0, None) == mxa.MX_EINVAL              # m_cap % 32
    assert w(P, Q, P, 2, 64, 64, 64, P, 0, None) == mxa.MX_EINVAL              # xt not 16-aligned
    assert w(P, P, P, 5000, 64, 64, 64, P, 0, None) == mxa.MX_EUNSUPPORTED


def test_swiglu_validation(lib):
    f = lib.mx_swiglu_quantize
    assert f(None, 64, 64, P, None, None, None, None, None) == mxa.MX_EINVAL             # h null
    assert f(P, 64, 48, P, None, None, None, None, None) == mxa.MX_EINVAL                # F % 32
    assert f(P, 64, 64, None, None, None, None, None, None) == mxa.MX_EINVAL             # no output
    assert f(P, 40, 64, None, None, None, P, P, None) == mxa.MX_EINVAL                   # colwise rows % 32
    assert f(P, 64, 64, None, P, None, None, None, None) == mxa.MX_EINVAL                # half a pair
    assert f(Q, 64, 64, P, None, None, None, None, None) == mxa.MX_EINVAL                # h alignment
    assert f(P, 0, 64, P, None, None, None, None, None) == mxa.MX_OK                     # empty
    b = lib.mx_swiglu_bwd_quantize
    assert b(P, None, 64, 64, P, None, None, None, None, None) == mxa.MX_EINVAL          # da null
    assert b(P, P, 64, 16, P, None, None, None, None, None) == mxa.MX_EINVAL             # F % 32
    assert b(P, P, 64, 64, None, None, None, None, None, None) == mxa.MX_EINVAL          # no output
    assert b(P, P, 0, 64, P, None, None, None, None, None) == mxa.MX_OK


def test_combine_validation(lib):
    c = lib.mx_combine
    assert c(None, 64, 64, P, P, 8, 2, P, None) == mxa.MX_EINVAL                         # y null
    assert c(P, 64, 48, P, P, 8, 2, P, None) == mxa.MX_EINVAL                            # H % 32
    assert c(P, 64, 64, P, P, 8, 0, P, None) == mxa.MX_EINVAL                            # topk 0
    assert c(P, 64, 64, None, P, 8, 2, P, None) == mxa.MX_EINVAL                         # dst null
    assert c(P, 64, 64, P, None, 0, 2, P, None) == mxa.MX_OK                             # no tokens
    b = lib.mx_combine_bwd_quantize
    assert b(P, None, P, P, 8, 2, 64, 64, P, None, None, None, None, None) == mxa.MX_EINVAL   # weights null
    assert b(P, P, P, P, 8, 2, 40, 64, None, None, None, P, P, None) == mxa.MX_EINVAL        # colwise rows % 32
    assert b(P, P, P, P, 8, 2, 64, 64, None, None, None, None, None, None) == mxa.MX_EINVAL  # no output
    assert b(P, P, P, P, 8, 2, 0, 64, P, None, None, None, None, None) == mxa.MX_OK


def test_router_validation(lib):
    r = lib.mx_route_topk
    assert r(None, 8, 16, 2, P, P, None) == mxa.MX_EINVAL                                 # logits null
    assert r(P, 8, 16, 0, P, P, None) == mxa.MX_EINVAL                                    # topk 0
    assert r(P, 8, 4, 5, P, P, None) == mxa.MX_EINVAL                                     # topk > E
    assert r(P, 8, 2048, 2, P, P, None) == mxa.MX_EUNSUPPORTED                            # E > 1024
    assert r(P, 0, 16, 2, P, P, None) == mxa.MX_OK                                        # no tokens
    b = lib.mx_router_bwd
    assert b(P, P, 64, 64, P, P, P, 8, 16, 2, None, None, None) == mxa.MX_EINVAL         # no output
    assert b(P, P, 64, 48, P, P, P, 8, 16, 2, P, None, None) == mxa.MX_EINVAL            # H % 32
    assert b(P, P, 64, 64, P, None, P, 8, 16, 2, None, P, None) == mxa.MX_EINVAL         # dlogits needs ids
    assert b(Q, P, 64, 64, P, P, P, 8, 16, 2, P, None, None) == mxa.MX_EINVAL            # alignment
    assert b(P, P, 64, 64, P, P, P, 0, 16, 2, P, P, None) == mxa.MX_OK


def test_python_binding_raises(lib):
    with pytest.raises(mxa.MXError):
        mxa.mx_dequantize(None, None, 4, 32, None, stream=0)


def test_permute_noalloc_validation(lib):
    """The no-allocation permute checks its arguments like mx_permute and
    rejects requests whose routing tables exceed its built-in scratch, all
    before touching the GPU."""
    p = lib.mx_permute_noalloc
    assert p(P, P, 100, 64, P, 2, 4, 200 + 31 * 4 - 1, P, P, P, P, P, None) == mxa.MX_EINVAL   # capacity
    assert p(P, P, 100, 64, P, 2, 4, 400, None, P, P, P, P, None) == mxa.MX_EINVAL             # half a copy
    assert p(Q, P, 100, 64, P, 2, 4, 400, P, P, P, P, P, None) == mxa.MX_EINVAL                # code alignment
    assert p(None, None, 100, 0, P, 0, 4, 400, None, None, P, P, P, None) == mxa.MX_EINVAL     # topk 0
    T, E = 1 << 18, 16384
    assert lib.mx_permute_workspace_size(T, 1, E) > (4 << 20)
    assert p(None, None, T, 0, P, 1, E, T + 31 * E, None, None, P, P, P, None) == mxa.MX_EUNSUPPORTED


def test_ceiling_validation(lib):
    c = lib.mx_ceiling_copy
    assert c(None, P, 4096, None) == mxa.MX_EINVAL                                 # src null
    assert c(P, P, 4096 + 16, None) == mxa.MX_EINVAL                               # bytes % 4096
    assert c(P, P, 0, None) == mxa.MX_EINVAL                                       # empty
    assert c(Q, P, 4096, None) == mxa.MX_EINVAL                                    # src not 16-aligned
    m = lib.mx_ceiling_mfma
    assert m(None, 1, 1, 1, None) == mxa.MX_EINVAL                                 # out null
    assert m(P, 0, 1, 1, None) == mxa.MX_EINVAL                                    # no workgroups
    t = lib.mx_ceiling_tile_pattern
    assert t(None, P, P, 128, 128, None) == mxa.MX_EINVAL                          # x null
    assert t(P, P, P, 96, 128, None) == mxa.MX_EINVAL                              # rows % 128
    assert t(P, P, P, 128, 160, None) == mxa.MX_EINVAL                             # cols % 128
    assert t(P, Q, P, 128, 128, None) == mxa.MX_EINVAL                             # row_out not 16-aligned
