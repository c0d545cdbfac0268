"""Oracle: dynamic fake quantize-dequantize (QDQ) of one FP32 tile.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this
module; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg use the oracle.

Sources ("[1/4] GDN state/W QAT foundation", section "What does this PR do?";
"[2/4] GDN/KDA decode QAT with INT8 recurrent state", sections "What does this
PR do?" and "Testing"):
  * dynamic scales (no calibration), FP8 E4M3 or signed symmetric INT8 with
    zero point zero, codes in [-127, 127], nearest-even rounding;
  * division by the scale is carried out as multiplication by the
    FP32-rounded reciprocal ("rounded reciprocal multiplication", [2/4]
    Testing).

Reading taken where the pages are silent:
  a   = max |x| over the tile                      (FP32)
  d   = fl32(a / q_max), floored at 2**-126        (q_max = 448 or 127)
  r   = fl32(1 / d)
  y_i = fl32(x_i * r)
  c_i = round-to-nearest-even of y_i onto the code grid
        E4M3 = OCP E4M3FN (bias 7, 3 mantissa bits, subnormal step 2**-9,
        largest finite 448, saturating, never NaN); INT8 = integers,
        clamped to [-127, 127]
  out = fl32(c_i * d)
A zero tile gives d = 2**-126 and returns zeros (signs kept).

All arithmetic here is numpy float32 (IEEE, round-to-nearest-even) except
the grid rounding, which is done exactly in float64 (a float32 divided by a
power of two is exact in float64).
"""
import numpy as np

FMT_OFF = 0
FMT_E4M3 = 1
FMT_INT8 = 2

E4M3_MAX = 448.0
INT8_MAX = 127.0
SCALE_FLOOR = np.float32(2.0 ** -126)


def qmax_of(fmt):
    if fmt == FMT_E4M3:
        return np.float32(E4M3_MAX)
    if fmt == FMT_INT8:
        return np.float32(INT8_MAX)
    raise ValueError(f"no code grid for format {fmt}")


def round_e4m3(y):
    """Round float32 values to the nearest OCP E4M3FN value, ties to even
    mantissa, saturating at +-448. Returns float32 (every E4M3 value is
    exactly representable)."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.abs(y64)
    # binade exponent e with 2**e <= a < 2**(e+1); frexp gives a = m * 2**x,
    # m in [0.5, 1), so e = x - 1. Below the smallest normal (2**-6) the grid
    # is the subnormal grid with step 2**-9, i.e. the e = -6 grid.
    _, x = np.frexp(a)
    e = np.maximum(x.astype(np.int64) - 1, -6)
    step = np.ldexp(1.0, e - 3)          # 3 mantissa bits
    c = np.rint(y64 / step) * step       # exact scaling, rint is ties-to-even
    c = np.clip(c, -E4M3_MAX, E4M3_MAX)  # saturate
    c = np.where(a == 0.0, y64, c)       # keep signed zeros
    return c.astype(np.float32)


def round_int8(y):
    """Round to the nearest integer, ties to even, clamped to [-127, 127]."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    c = np.clip(np.rint(y64), -INT8_MAX, INT8_MAX)
    return c.astype(np.float32)


def round_codes(y, fmt):
    if fmt == FMT_E4M3:
        return round_e4m3(y)
    if fmt == FMT_INT8:
        return round_int8(y)
    raise ValueError(f"no code grid for format {fmt}")


def scale_of(amax, fmt):
    """d = max(fl32(amax / q_max), 2**-126) in float32."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(under="ignore"):
        d = (amax / qmax_of(fmt)).astype(np.float32)
    return np.maximum(d, SCALE_FLOOR).astype(np.float32)


def qdq32(x, fmt, tile_axes):
    """Fake-quantize float32 array `x` with one scale per tile; a tile is
    the set of elements sharing all indices outside `tile_axes`.

    Returns (out, codes, d): out and codes have x's shape (float32), d has
    x's shape with `tile_axes` reduced to length 1 (float32)."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == FMT_OFF:
        return x.copy(), None, None
    amax = np.max(np.abs(x), axis=tile_axes, keepdims=True)
    d = scale_of(amax, fmt)
    r = (np.float32(1.0) / d).astype(np.float32)
    y = (x * r).astype(np.float32)
    c = round_codes(y, fmt)
    out = (c * d).astype(np.float32)
    return out, c, d


# ---------------------------------------------------------------------------
# OCP E4M3FN bit encoding, used to compare exported one-byte codes.
# Layout: sign(1) exponent(4, bias 7) mantissa(3); exponent 0 = subnormal
# (value m/8 * 2**-6); 0x7F / 0xFF are NaN; no infinities.
# ---------------------------------------------------------------------------

def e4m3_decode_table():
    """float64 value of each of the 256 byte codes (NaN for 0x7F, 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for b in range(256):
        s = -1.0 if (b >> 7) & 1 else 1.0
        ex = (b >> 3) & 0xF
        m = b & 0x7
        if ex == 0xF and m == 0x7:
            vals[b] = np.nan
        elif ex == 0:
            vals[b] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[b] = s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return vals


def e4m3_encode(c):
    """Byte code of float values that lie exactly on the E4M3 grid."""
    table = e4m3_decode_table()[:0x7F]   # codes 0x00..0x7E, strictly increasing
    c = np.asarray(c, dtype=np.float64)
    a = np.abs(c)
    idx = np.searchsorted(table, a)
    if not np.array_equal(table[np.minimum(idx, 0x7E)], a):
        raise ValueError("value not on the E4M3 grid")
    sign = np.signbit(c).astype(np.int64) << 7
    return (idx.astype(np.int64) | sign).astype(np.uint8)
