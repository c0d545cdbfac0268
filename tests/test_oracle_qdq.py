"""Pins of the oracle's FP32 QDQ function against definitions that do not
share its arithmetic: brute-force nearest-code search over the decoded E4M3
table and over the integers, idempotence, the max-code invariant, and the
rounding error bound.

Contract pinned ("[1/4] GDN state/W QAT foundation", "What does this PR do?":
dynamic E4M3; "[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What
does this PR do?": INT8 codes in [-127, 127], zero point zero, nearest-even;
"Testing": rounded reciprocal multiplication)."""
import numpy as np
import pytest

from oracle.qdq import (FMT_E4M3, FMT_INT8, e4m3_decode_table, e4m3_encode, qdq32,
                        round_e4m3, round_int8)


def _stratified_f32():
    """Every sign x exponent x top-12 mantissa bits, each with five patterns
    of the low 11 mantissa bits (exact ties, just above/below): all rounding
    decisions of a grid with <= 12 mantissa bits are exercised."""
    exps = np.arange(0, 140, dtype=np.uint32)            # |y| < 2**13
    top = np.arange(4096, dtype=np.uint32)
    low = np.array([0, 1, 0x3FF, 0x400, 0x7FF], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | (top[None, :, None] << 11) | low[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def _brute_nearest(y, grid, code_is_even):
    """Nearest value of a sorted grid (ties -> even code), by searching."""
    y = y.astype(np.float64)
    idx = np.searchsorted(grid, y)
    lo = np.clip(idx - 1, 0, len(grid) - 1)
    hi = np.clip(idx, 0, len(grid) - 1)
    dlo = np.abs(y - grid[lo])
    dhi = np.abs(grid[hi] - y)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                    np.where(code_is_even[lo], lo, hi)))
    return grid[pick]


def test_e4m3_table():
    t = e4m3_decode_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    fin = t[~np.isnan(t)]
    assert fin.size == 254
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert np.all(np.diff(t[:0x7F]) > 0)
    # round trip of every finite code
    codes = np.array([b for b in range(256) if not np.isnan(t[b])], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(t[codes]), codes)


def test_round_e4m3_matches_bruteforce():
    t = e4m3_decode_table()
    pos = t[:0x7F]                                      # 0 .. 448
    grid = np.concatenate([-pos[::-1][:-1], pos])       # -448 .. 448
    codes = np.concatenate([np.arange(0x7E, 0, -1), np.arange(0, 0x7F)])
    even = (codes & 1) == 0
    y = _stratified_f32()
    got = round_e4m3(y).astype(np.float64)
    want = _brute_nearest(y, grid, even)
    bad = got != want
    assert not bad.any(), (y[bad][:5], got[bad][:5], want[bad][:5])


def test_round_int8_matches_bruteforce():
    grid = np.arange(-127, 128, dtype=np.float64)
    even = (np.arange(-127, 128) % 2) == 0
    y = _stratified_f32()
    y = y[np.abs(y) < 300]
    got = round_int8(y).astype(np.float64)
    want = _brute_nearest(y, grid, even)
    np.testing.assert_array_equal(got, want)


def _tiles(rng, n=400):
    """Random [16, 32] tiles over many magnitudes and shapes."""
    out = []
    for i in range(n):
        kind = i % 5
        x = rng.standard_normal((16, 32))
        if kind == 1:
            x = x ** 3                                     # heavy tails
        elif kind == 2:
            x = x * 1e-40                                  # subnormal FP32 inputs
        elif kind == 3:
            x = np.where(rng.random((16, 32)) < 0.5, 0.0, x) * 1e6
        elif kind == 4:
            x = rng.integers(-8, 9, (16, 32)) * 2.0 ** rng.integers(-20, 20)
        out.append(x.astype(np.float32) * np.float32(2.0 ** rng.integers(-30, 30)))
    return np.stack(out)


@pytest.mark.parametrize("fmt", [FMT_E4M3, FMT_INT8])
def test_qdq_idempotent_bitexact(fmt):
    x = _tiles(np.random.default_rng(1))
    y, _, _ = qdq32(x, fmt, (1, 2))
    z, _, _ = qdq32(y, fmt, (1, 2))
    np.testing.assert_array_equal(y.view(np.uint32), z.view(np.uint32))


@pytest.mark.parametrize("fmt,qmax", [(FMT_E4M3, 448.0), (FMT_INT8, 127.0)])
def test_qdq_max_code_and_error_bound(fmt, qmax):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 8, 64)).astype(np.float32) * np.float32(3.0)
    out, c, d = qdq32(x, fmt, (1, 2))
    a = np.abs(x).max(axis=(1, 2), keepdims=True)
    # the amax element lands on the largest code
    at_max = np.abs(x) == a
    assert np.all(np.abs(c[at_max]) == qmax)
    # scale is amax / qmax rounded to FP32
    np.testing.assert_array_equal(d, (a / np.float32(qmax)).astype(np.float32))
    y = x.astype(np.float64) / d.astype(np.float64)
    err = np.abs(c.astype(np.float64) - y)
    if fmt == FMT_E4M3:
        bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
    else:
        bound = 0.5 + 1e-4
    assert np.all(err <= bound)


def test_qdq_zero_tile_and_signs():
    x = np.zeros((2, 4, 8), np.float32)
    x[0, 0, 0] = -0.0
    x[1] = np.float32(-0.0)
    for fmt in (FMT_E4M3, FMT_INT8):
        out, c, d = qdq32(x, fmt, (1, 2))
        np.testing.assert_array_equal(out.view(np.uint32), x.view(np.uint32))
        assert np.all(d == np.float32(2.0 ** -126))


def test_qdq_tiles_are_independent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 16, 2, 8)).astype(np.float32)   # [H, Dk, nb, bv]
    out, _, d = qdq32(x, FMT_E4M3, (1, 3))
    assert d.shape == (4, 1, 2, 1)
    x2 = x.copy()
    x2[:, :, 1, :] *= 1000.0                                      # other tile only
    out2, _, _ = qdq32(x2, FMT_E4M3, (1, 3))
    np.testing.assert_array_equal(out[:, :, 0], out2[:, :, 0])


def _reciprocal_fixture():
    import json
    import os
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'golden', 'qdq_reciprocal.json')
    return json.load(open(p))['tiles']


def test_qdq_uses_rounded_reciprocal():
    """y = x * fl32(1/d), not x / d ("[2/4] GDN/KDA decode QAT with INT8
    recurrent state", "Testing": rounded reciprocal multiplication). The
    fixture tiles (tests/golden/make_qdq_reciprocal.py) hold, for both
    formats and non-power-of-two scales, 40 values each whose codes differ
    between the two forms; the oracle must give the reciprocal-form codes on
    every element, which plain division misses on those 40."""
    tiles = _reciprocal_fixture()
    assert {t['fmt'] for t in tiles} == {FMT_E4M3, FMT_INT8}
    for t in tiles:
        x = np.array(t['x_bits'], np.uint32).view(np.float32)[None]
        out, c, d = qdq32(x, t['fmt'], (1,))
        assert np.array(d[0, 0], np.float32).view(np.uint32) == t['d_bits']
        np.testing.assert_array_equal(c[0], np.float32(t['codes']))
        # the stored codes separate the two conventions on many elements
        differ = np.float32(t['codes']) != np.float32(t['div_codes'])
        assert differ.sum() >= 30, differ.sum()
        # and the division form really gives the other codes on this input
        dd = np.float32(d[0, 0])
        c_div = round_e4m3((x[0] / dd).astype(np.float32)) if t['fmt'] == FMT_E4M3 else \
            np.clip(np.rint((x[0] / dd).astype(np.float32).astype(np.float64)), -127, 127)
        np.testing.assert_array_equal(np.float32(c_div)[differ], np.float32(t['div_codes'])[differ])
        assert np.all(np.float32(c_div)[differ] != c[0][differ])
