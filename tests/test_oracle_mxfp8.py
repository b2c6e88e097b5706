"""Pins for the MXFP8 codec oracle (CPU only).

Each test checks the oracle against something other than itself: torch's
independent float8 codecs, brute-force nearest-value search, hand-derived
golden blocks, closed forms and invariants.  Format: OCP MX (E4M3 elements,
E8M0 block scales of 32), the microscaling scheme of the MXFP8 MoE digest
("Key Questions Answered").
"""

import json
import os
import struct

import numpy as np
import pytest
import torch

from oracle import mxfp8 as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e8m0(b):
    return torch.from_numpy(np.asarray(b, np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def f32_bits_to_bf16(vals):
    return np.array([struct.unpack("<I", struct.pack("<f", v))[0] >> 16 for v in vals], dtype=np.uint16)


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256)
    ours, ref = mx.e4m3_decode(codes), torch_e4m3(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3_fixed_facts():
    d = mx.e4m3_decode
    assert d(0x7E) == 448.0 and np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x01) == 2.0 ** -9 and d(0x08) == 2.0 ** -6 and d(0x38) == 1.0
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    pos = d(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0) and pos.size == 127


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def brute_force_e4m3(v):
    """Nearest of the 127 non-negative finite E4M3 magnitudes, ties to the even
    code (= even mantissa); sign applied afterwards."""
    mags = torch_e4m3(np.arange(0x7F))            # independent decode
    a = np.abs(v)[:, None]
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    n_c = cand.sum(axis=1)
    first = np.argmax(cand, axis=1)
    last = 126 - np.argmax(cand[:, ::-1], axis=1)
    code = np.where(n_c == 1, first, np.where(first % 2 == 0, first, last))
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_e4m3_encode_exhaustive_bf16_times_scale():
    """Every finite bf16 value times every scale 2^-s, s in [-127, 127]:
    the oracle encoder equals brute-force nearest search (distinct values
    are deduplicated first; there are ~80k of them)."""
    bits = np.arange(0x7F80, dtype=np.uint16)            # positive finite bf16
    x = mx.bf16_to_f64(bits)
    vals = np.unique(np.concatenate([np.ldexp(x, -s) for s in range(-127, 128)]))
    ours = mx.e4m3_encode(vals)
    # fp64 distances are exact while |v| < 2^40 (8 + 4 significant bits);
    # beyond that every value is nearest to 448.
    small = vals < 2.0 ** 40
    assert np.all(ours[~small] == 0x7E)
    vs, os_ = vals[small], ours[small]
    for lo in range(0, vs.size, 20000):
        sl = slice(lo, lo + 20000)
        assert np.array_equal(os_[sl], brute_force_e4m3(vs[sl]))
    neg = mx.e4m3_encode(-vals)
    assert np.array_equal(neg, ours | 0x80)


def test_e4m3_encode_vs_torch_below_448():
    g = np.random.default_rng(7)
    v = np.concatenate([g.standard_normal(200000) * 10.0 ** g.uniform(-4, 2.5, 200000),
                        mx.e4m3_decode(np.arange(0x7E)) + np.ldexp(1.0, -30)])
    v = v[np.abs(v) < 448]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mx.e4m3_encode(v.astype(np.float32).astype(np.float64)), ref)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 463.9, 464.0, 479.0, 480.0, 512.0, 1e9, -464.0, -1e30])
    assert list(mx.e4m3_encode(v)) == [0x7E] * 7 + [0xFE, 0xFE]
    with pytest.raises(ValueError):
        mx.e4m3_encode(np.array([np.nan]))


def test_e8m0_decode_vs_torch_and_zero_byte():
    b = np.arange(256)
    ours, ref = mx.e8m0_decode(b), torch_e8m0(b)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[:255], ref[:255])
    assert mx.e8m0_decode(0) == 2.0 ** -127 and mx.e8m0_decode(127) == 1.0


def test_scale_byte_fixed_facts():
    f = mx.e8m0_scale_byte
    assert f(448.0) == 127           # the build target's fixed fact: amax 448 -> 2^0
    assert f(1.0) == 119 and f(511.99) == 127 and f(512.0) == 128 and f(447.0) == 127
    assert f(0.0) == 0 and f(2.0 ** -120) == 0 and f(2.0 ** -118) == 1
    assert f(2.0 ** -133) == 0       # bf16 subnormal amax
    assert f(mx.bf16_to_f64(0x7F7F)) == 246   # largest finite bf16 never reaches the upper clamp


def test_golden_blocks():
    with open(os.path.join(GOLDEN, "quant_blocks.json")) as fh:
        blocks = json.load(fh)["blocks"]
    rows, want_q, want_s = [], [], []
    for b in blocks:
        if "values" in b:
            rows.append(f32_bits_to_bf16(b["values"]))
        else:
            rows.append(np.array([int(h, 16) for h in b["bf16_bits"]], np.uint16))
        want_q.append([int(h, 16) for h in b["codes"]])
        want_s.append(b["scale_byte"])
    q, s = mx.quantize_rowwise(np.stack(rows))
    assert np.array_equal(s[:, 0], np.array(want_s, np.uint8))
    assert np.array_equal(q, np.array(want_q, np.uint8))


def random_bf16_blocks(n, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, 32)).astype(np.float32)
    x *= (10.0 ** g.uniform(-30, 30, (n, 1))).astype(np.float32)
    x[g.random((n, 32)) < 0.01] *= 1000
    x[g.random(n) < 0.05] = 0
    b = f32_bits_to_bf16(x.ravel()).reshape(n, 32)
    sub = g.random(n) < 0.05
    b[sub] = g.integers(0, 128, (int(sub.sum()), 32)).astype(np.uint16) | (g.integers(0, 2, (int(sub.sum()), 32)).astype(np.uint16) << 15)
    return b


def test_quantize_invariants_random_blocks():
    """Scale off by one in either direction breaks the max-code window;
    a wrong rounding breaks the half-ulp error bound."""
    b = random_bf16_blocks(20000, 3)
    x = mx.bf16_to_f64(b)
    q, s = mx.quantize_rowwise(b)
    s = s[:, 0].astype(np.int64)
    amax = np.abs(x).max(1)
    normal = (s > 0) & (amax > 0)
    maxcode = (q & 0x7F).max(1)
    assert np.all((maxcode[normal] >= 0x78) & (maxcode[normal] <= 0x7E))
    zero = amax == 0
    assert np.all(s[zero] == 0) and np.all(q[zero] == 0)
    scaled = np.ldexp(x, -(s[:, None] - 127))
    back = mx.e4m3_decode(q)
    sat = np.abs(scaled) >= 448
    assert np.all((q[sat] & 0x7F) == 0x7E)
    a = np.abs(scaled[~sat])
    _, e = np.frexp(a)
    half_ulp = np.ldexp(1.0, np.maximum(e - 1, -6) - 4)
    assert np.all(np.abs(back[~sat] - scaled[~sat]) <= half_ulp)
    assert np.all(np.signbit(back[~sat]) == np.signbit(scaled[~sat]))


def test_quantize_requantize_idempotent():
    b = random_bf16_blocks(5000, 11)
    q, s = mx.quantize_rowwise(b)
    y = mx.dequantize(q, s)
    exact = mx.bf16_to_f64(y) == mx.mx_values(q, s)
    rows = exact.all(axis=1)
    q2, s2 = mx.quantize_rowwise(y[rows])
    assert rows.sum() > 4000
    assert np.array_equal(q2, q[rows]) and np.array_equal(s2, s[rows])


def test_dequantize_exhaustive_vs_torch():
    """256 codes x 256 scale bytes.  The fp32 product of an E4M3 value and a
    power of two is exact (or overflows), so torch's fp32->bf16 rounding is
    an independent reference here."""
    c, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    c = c.astype(np.uint8)
    b = b.astype(np.uint8)
    q = np.repeat(c.reshape(-1, 1), 32, axis=1)
    ours = mx.dequantize(q, b.reshape(-1, 1))[:, 0]
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (torch_e4m3(c.ravel()) * torch_e8m0(b.ravel())).astype(np.float32)
    ref = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(prod)
    assert np.array_equal(np.isnan(mx.bf16_to_f64(ours)), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f64_to_bf16_direct_rounding():
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8 + 2.0 ** -40),
                  2.0 ** -134, 2.0 ** -134 + 2.0 ** -160, 3 * 2.0 ** -134, 3.3895313892515355e38, 3.4e38, 0.0, -0.0])
    want = [0x3F80, 0x3F82, 0x3F81, 0xBF81, 0x0000, 0x0001, 0x0002, 0x7F7F, 0x7F80, 0x0000, 0x8000]
    assert list(mx.f64_to_bf16(v)) == want
    g = np.random.default_rng(5)
    f = (g.standard_normal(100000) * 10.0 ** g.uniform(-45, 38, 100000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx.f64_to_bf16(f.astype(np.float64)), ref)


def test_colwise_hand_built():
    """Column c of rows 0..31 is (r+1) * 2^(c-10): every column block is the
    golden ramp, so codes equal the ramp's and the byte is 124 + c - 10; rows
    32..63 are zero (byte 0)."""
    with open(os.path.join(GOLDEN, "quant_blocks.json")) as fh:
        ramp = json.load(fh)["blocks"][0]
    ramp_codes = np.array([int(h, 16) for h in ramp["codes"]], np.uint8)
    vals = np.zeros((64, 32), np.float32)
    for c in range(32):
        vals[:32, c] = (np.arange(32) + 1) * 2.0 ** (c - 10)
    b = f32_bits_to_bf16(vals.ravel()).reshape(64, 32)
    qt, st = mx.quantize_colwise(b)
    assert qt.shape == (32, 64) and st.shape == (32, 2)
    for c in range(32):
        assert np.array_equal(qt[c, :32], ramp_codes)
        assert st[c, 0] == 124 + c - 10
    assert np.all(qt[:, 32:] == 0) and np.all(st[:, 1] == 0)
    # gather: reversed rows with a zero row slot; rows_out padded to 96
    gather = np.concatenate([np.arange(31, -1, -1), [-1] * 32, np.arange(32)])
    qg, sg = mx.quantize_colwise(b, rows_out=96, gather=gather)
    assert np.array_equal(qg[:, :32], qt[:, :32][:, ::-1])
    assert np.all(qg[:, 32:64] == 0) and np.all(sg[:, 1] == 0)
    assert np.array_equal(qg[:, 64:], qt[:, :32]) and np.array_equal(sg[:, 2], st[:, 0])


def test_colwise_padding_invariance():
    """A group's last partial block computed over its real rows only equals the
    block of the zero-padded layout."""
    g = np.random.default_rng(9)
    x = f32_bits_to_bf16(g.standard_normal(50 * 64).astype(np.float32)).reshape(50, 64)
    qt, st = mx.quantize_colwise(x, rows_out=64)
    part = x[32:50]                                   # 18 real rows of the second block
    amax = np.abs(mx.bf16_to_f64(part)).max(axis=0)
    assert np.array_equal(st[:, 1], mx.e8m0_scale_byte(amax))
    codes = mx.e4m3_encode(np.ldexp(mx.bf16_to_f64(part), 127 - st[:, 1].astype(np.int64)[None, :]))
    assert np.array_equal(qt[:, 32:50], codes.T) and np.all(qt[:, 50:] == 0)
