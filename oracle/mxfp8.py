"""Oracle: OCP MXFP8 element and scale codecs, quantize and dequantize.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain NumPy; every
real-valued step is done in fp64, where the operations used here are exact.

Format (microscaling, digest page "Key Questions Answered": a scale per
fine-grained sub-block; numeric rules per OCP MX v1.0 as restated by the
build target):

* element: E4M3 "fn" -- 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
  infinities, NaN = S.1111.111, largest finite 448, smallest subnormal 2^-9;
* scale: E8M0 -- an unsigned biased exponent, value 2^(byte-127), byte 255
  is NaN, byte 0 is 2^-127 (NOT zero);
* block: 32 consecutive elements along the quantized axis share one scale.

bf16 values are carried as their uint16 bit patterns.
"""

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest E4M3 power of two (448 = 1.75 * 2^8)
E8M0_BIAS = 127


# --------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------
def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns (the top half of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """Round fp64 values to bf16 bit patterns: round to nearest, ties to even,
    gradual underflow (bf16 subnormals kept, no flush), overflow to +-Inf,
    NaN -> 0x7FC0.

    Written from the definition: the bf16 grid near |v| has quantum
    2^(e-7), e = max(floor(log2|v|), -126); |v| is scaled onto that grid,
    rounded half-to-even, and scaled back.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, x = np.frexp(a)            # a = f * 2^x, f in [0.5, 1)
    e = np.maximum(x - 1, -126)   # floor(log2 a) clamped to the subnormal exponent
    n = np.ldexp(a, 7 - e)        # a / quantum, exact
    r = np.rint(n)                # ties to even
    mag = np.ldexp(r, e - 7)
    with np.errstate(over="ignore"):
        bits = (mag.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.signbit(v), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(v), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# --------------------------------------------------------------------------
# E4M3 and E8M0
# --------------------------------------------------------------------------
def e4m3_decode(codes):
    """Value of E4M3 codes (fp64).  0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_encode(v):
    """Round fp64 values to E4M3 codes: nearest, ties to the even mantissa,
    saturating (|v| >= 448 -> 448).  The sign is kept, so -0 and negative
    values that round to zero give 0x80.

    The rounding grid has quantum 2^(e-3) with e = max(floor(log2|v|), -6):
    three mantissa bits in the normal range, a fixed 2^-9 step in the
    subnormal range.  NaN and infinite inputs are outside the contract and
    raise.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(v)
    _, x = np.frexp(a)
    e = np.maximum(x - 1, -6)
    r = np.rint(np.ldexp(a, 3 - e))          # in [0, 16]; ties to even
    carry = r == 16                          # rounded up into the next binade
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r).astype(np.int64)
    code = np.where(r < 8, r, ((e + 7) << 3) + (r - 8))   # r < 8 only in the subnormal range
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code.astype(np.int64) | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def e8m0_decode(byte):
    """Value 2^(byte-127) of E8M0 scale bytes; byte 255 is NaN, byte 0 is 2^-127."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def e8m0_scale_byte(amax):
    """Shared-scale byte of a block with absolute maximum ``amax``.

    Scale exponent = floor(log2(amax)) - 8, clamped to the E8M0 range
    [-127, 127]; an all-zero block (amax = 0, log2 = -inf) clamps to -127,
    i.e. byte 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(a)
    s = np.where(a > 0, (x - 1) - E4M3_EMAX, -E8M0_BIAS)
    s = np.clip(s, -E8M0_BIAS, E8M0_BIAS)
    return (s + E8M0_BIAS).astype(np.uint8)


# --------------------------------------------------------------------------
# quantize / dequantize
# --------------------------------------------------------------------------
def quantize_rowwise(x_bits):
    """MXFP8-quantize a bf16 matrix along its last axis.

    ``x_bits``: uint16 [..., C] with C a multiple of 32.  Returns
    (q uint8 [..., C], s uint8 [..., C/32]); block b of row r covers columns
    [32b, 32b+32).  q = E4M3(x * 2^-scale_exponent), exact in fp64 because
    the scale is a power of two.
    """
    x = bf16_to_f64(x_bits)
    C = x.shape[-1]
    if C % BLOCK:
        raise ValueError("quantize_rowwise: last dimension must be a multiple of 32")
    xb = x.reshape(*x.shape[:-1], C // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)
    s = e8m0_scale_byte(amax)
    q = e4m3_encode(np.ldexp(xb, E8M0_BIAS - s.astype(np.int64)[..., None]))
    return q.reshape(x.shape), s


def gather_rows(x_bits, gather, rows_out):
    """Rows of the (zero-padded) source selected for a columnwise quantize:
    output row r is source row ``gather[r]``, or a zero row when
    ``gather[r] < 0``; without a gather, output row r is source row r and
    rows past the source are zero."""
    x = np.asarray(x_bits, dtype=np.uint16)
    R, C = x.shape
    out = np.zeros((rows_out, C), dtype=np.uint16)
    if gather is None:
        n = min(R, rows_out)
        out[:n] = x[:n]
    else:
        g = np.asarray(gather, dtype=np.int64)[:rows_out]
        ok = g >= 0
        out[:len(g)][ok] = x[g[ok]]
    return out


def quantize_colwise(x_bits, rows_out=None, gather=None):
    """MXFP8-quantize a bf16 matrix along its rows (blocks of 32 consecutive
    rows within one column) and store the result transposed.

    ``x_bits`` uint16 [R, C]; ``rows_out`` a multiple of 32 (default R);
    optional ``gather`` int [rows_out] selects the source row of each output
    row (-1 = zero row).  Returns (qT uint8 [C, rows_out],
    sT uint8 [C, rows_out/32]): qT[c, r] is the code of element (r, c) and
    sT[c, b] the scale of rows [32b, 32b+32) of column c.

    Groups of rows (experts) never share a block because every group starts
    at a multiple of 32 in the padded layout and pad rows are zero; zero rows
    change neither a block's amax nor any code.
    """
    x = np.asarray(x_bits, dtype=np.uint16)
    if rows_out is None:
        rows_out = x.shape[0]
    if rows_out % BLOCK:
        raise ValueError("quantize_colwise: rows_out must be a multiple of 32")
    xr = gather_rows(x, gather, rows_out)
    return quantize_rowwise(np.ascontiguousarray(xr.T))


def dequantize(q, s):
    """bf16 bit patterns of decode(q) * 2^(s-127), rounded to nearest even
    (subnormals kept, overflow to Inf).  Blocks of 32 along the last axis.
    A code 0x7F/0xFF or a scale byte 255 gives NaN."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    C = q.shape[-1]
    vals = e4m3_decode(q).reshape(*q.shape[:-1], C // BLOCK, BLOCK)
    y = vals * e8m0_decode(s)[..., None]
    return f64_to_bf16(y.reshape(q.shape))


def mx_values(q, s):
    """fp64 values represented by an MX tensor (blocks of 32 along the last axis)."""
    q = np.asarray(q, dtype=np.uint8)
    C = q.shape[-1]
    vals = e4m3_decode(q).reshape(*q.shape[:-1], C // BLOCK, BLOCK)
    return (vals * e8m0_decode(np.asarray(s))[..., None]).reshape(q.shape)
