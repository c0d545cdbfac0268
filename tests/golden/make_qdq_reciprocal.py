"""Writes tests/golden/qdq_reciprocal.json: QDQ tiles on which the
rounded-reciprocal multiply and plain division give different codes.

"[2/4] GDN/KDA decode QAT with INT8 recurrent state", section "Testing": the
division of a value by its tile scale d is carried out as a multiplication
by the FP32-rounded reciprocal fl32(1/d), as Torch's scalar division does.
On random tiles the two forms round to different codes only a few times per
million values, so random inputs cannot tell them apart. The tiles here are
built so that they do: for a tile maximum a (not a power of two times the
grid maximum), d = fl32(a / q_max) and r = fl32(1 / d); for every grid
midpoint m below q_max the FP32 neighbours of fl32(m d) are tried, and a
value x is kept when RNE(fl32(x r)) and RNE(fl32(x / d)) are different codes.
Each tile is [a, kept values..., zeros] (a stays the tile maximum, so d is
the same for every element).

Stored per tile: the FP32 bit patterns of the inputs, the oracle's codes and
scale (oracle.qdq.qdq32, the only source of expected values) and, for
reference, the codes plain division would give. Run from the repo root:
    python tests/golden/make_qdq_reciprocal.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle.qdq import FMT_E4M3, FMT_INT8, qdq32, qmax_of, round_codes, scale_of  # noqa: E402

TILE = 256          # one [16, 16] state tile
PER_TILE = 40       # values that tell the two forms apart, per tile
TILES_PER_FMT = 4


def grid_midpoints(fmt):
    if fmt == FMT_INT8:
        return np.arange(0, 127, dtype=np.float64) + 0.5
    # E4M3FN grid values 0 .. 448 (subnormal step 2^-9, 3 mantissa bits)
    vals = [m / 8.0 * 2.0 ** -6 for m in range(8)]
    for e in range(-6, 9):
        for m in range(8):
            v = (1.0 + m / 8.0) * 2.0 ** e
            if v <= 448.0:
                vals.append(v)
    vals = np.array(sorted(set(vals)))
    return (vals[:-1] + vals[1:]) / 2.0


def search_tile(fmt, amax):
    """Values x < amax (FP32) whose codes under x * fl32(1/d) and x / d differ."""
    a32 = np.float32(amax)
    d = scale_of(a32, fmt)
    r = (np.float32(1.0) / d).astype(np.float32)
    found = []
    for m in grid_midpoints(fmt):
        x0 = np.float32(m * float(d))
        bits = np.array([x0], np.float32).view(np.uint32)[0]
        cand = (np.arange(-3, 4, dtype=np.int64) + int(bits)).astype(np.uint32).view(np.float32)
        for sgn in (1.0, -1.0):
            xs = (cand * np.float32(sgn)).astype(np.float32)
            xs = xs[np.abs(xs) < a32]
            y_mul = (xs * r).astype(np.float32)
            y_div = (xs / d).astype(np.float32)
            diff = round_codes(y_mul, fmt) != round_codes(y_div, fmt)
            found.extend(xs[diff].tolist())
    return np.array(found, np.float32)


def build():
    rng = np.random.default_rng(20251203)
    out = []
    for fmt in (FMT_E4M3, FMT_INT8):
        made = 0
        while made < TILES_PER_FMT:
            amax = np.float32(rng.uniform(0.5, 8.0))
            q = float(amax) / float(qmax_of(fmt))
            if np.log2(q) == np.round(np.log2(q)):
                continue                             # d must not be a power of two
            vals = search_tile(fmt, amax)
            if vals.size < 8:
                continue
            vals = vals[rng.permutation(vals.size)[:PER_TILE]]
            tile = np.zeros(TILE, np.float32)
            tile[0] = amax
            tile[1:1 + vals.size] = vals
            _, c_or, d_or = qdq32(tile[None], fmt, (1,))
            c_div = round_codes((tile / d_or[0, 0]).astype(np.float32), fmt)
            out.append(dict(fmt=int(fmt), x_bits=[int(b) for b in tile.view(np.uint32)],
                            d_bits=int(np.array([d_or[0, 0]], np.float32).view(np.uint32)[0]),
                            codes=c_or[0].astype(np.float64).tolist(),
                            div_codes=c_div.astype(np.float64).tolist(),
                            n_differ=int(np.sum(c_or[0] != c_div))))
            made += 1
    return out


if __name__ == '__main__':
    tiles = build()
    with open(os.path.join(HERE, 'qdq_reciprocal.json'), 'w') as f:
        json.dump(dict(tiles=tiles), f)
    print('wrote qdq_reciprocal.json:', [(t['fmt'], t['n_differ']) for t in tiles])
