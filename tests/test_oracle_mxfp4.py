"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against the OCP MX format
tables (tests/golden/mxfp4_format_table.txt), an independent brute-force
nearest-value encoder, closed-form scale exponents and worked blocks."""

import math
import os

import numpy as np
import pytest

from oracle import mxfp4 as mx

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    rows = {}
    with open(os.path.join(HERE, "golden", "mxfp4_format_table.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows[parts[0]] = parts[1:]
    return rows


def test_e2m1_table_matches_the_specification():
    g = _golden()
    t = mx.decode_table()
    for name in ("zero", "min_subnormal", "min_normal", "one_and_half", "max_normal"):
        pattern, value = g[name]
        s, e, m = pattern.split(".")
        code = (int(s) << 3) | (int(e, 2) << 1) | int(m, 2)
        assert t[code] == float(value), name
        assert t[code | 0x8] == -float(value) or (float(value) == 0 and t[code | 0x8] == 0)
    # all 8 magnitudes, increasing
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert int(g["block_size"][0]) == mx.BLOCK


def test_e8m0_table_matches_the_specification():
    g = _golden()
    for name in ("scale_min", "scale_one", "scale_max"):
        code, value = g[name]
        assert mx.scale_value(int(code, 16)) == float(value), name
    assert math.isnan(mx.scale_value(int(g["scale_nan"][0], 16)))


def _brute_encode(y):
    """Nearest of the 16 codes by exhaustive distance (independent of the
    oracle's search): ties to the code with LSB 0, saturation at 6, NaN -> 0,
    the sign of zero kept."""
    y = float(y)
    if math.isnan(y):
        return 0
    neg = math.copysign(1.0, y) < 0
    mag = min(abs(y), 6.0)
    best = None
    for code in range(8):
        v = mx.decode_table()[code]
        d = abs(mag - v)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1] | (0x8 if neg else 0)


def _probe_values():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]
    vals = mags + mids + [6.5, 7.0, 8.0, 100.0, 1e-30, 0.1, 0.2, 0.3, 5.5, 5.999]
    v32 = np.array(vals, dtype=np.float32)
    up = np.nextafter(v32, np.float32(np.inf))
    dn = np.nextafter(v32, np.float32(-np.inf))
    rng = np.random.default_rng(0)
    rnd = rng.uniform(-9, 9, 4000).astype(np.float32)
    allv = np.concatenate([v32, -v32, up, -up, dn, -dn, rnd,
                           np.array([np.inf, -np.inf, np.nan, -0.0], dtype=np.float32)])
    return allv


def test_encode_equals_brute_force_nearest():
    y = _probe_values()
    codes = mx.encode_elements(y)
    ref = np.array([_brute_encode(v) for v in y], dtype=np.uint8)
    assert np.array_equal(codes, ref)


def test_encode_worked_ties_and_saturation():
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -0.0], dtype=np.float32)
    # ties go to the even code: 0, 1, 1, 2, 2, 4, 4; 7 saturates to 6; signs kept
    assert list(mx.encode_elements(y)) == [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x7, 0x8, 0x8]


@pytest.mark.parametrize("amax,code,flags", [
    (6.0, 127, 0),                    # floor(log2 6) = 2 -> X = 1
    (7.9, 127, 0),
    (8.0, 128, 0),                    # 3 - 2 = 1
    (0.75, 124, 0),                   # -1 - 2 = -3
    (1.0, 125, 0),
    (np.float32(3.4028235e38), 252, 0),   # 127 - 2
    (np.float32(2.0 ** -130), 0, 0),  # subnormal amax: -130 - 2 clamped to -127
    (np.float32(2.0 ** -120), 5, 0),  # -120 - 2 = -122, inside the E8M0 range
    (0.0, 127, mx.FLAG_ZERO_AMAX),
    (np.inf, 0xFF, mx.FLAG_NONFINITE),
    (np.nan, 0xFF, mx.FLAG_NONFINITE),
])
def test_scale_exponent_closed_forms(amax, code, flags):
    assert mx.scale_exponent(amax) == (code, flags)


def test_block_roundtrip_error_bound_and_exact_grid():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, 128)) * np.exp(rng.standard_normal((8, 1)))).astype(np.float32)
    codes, scales, flags = mx.quantize(W)
    assert flags == 0 and codes.shape == (8, 64) and scales.shape == (8, 4)
    What = mx.dequantize(codes, scales)
    for i in range(8):
        for b in range(4):
            blk = W[i, 32 * b:32 * (b + 1)].astype(np.float64)
            X = mx.scale_value(scales[i, b])
            am = np.abs(blk).max()
            # X = 2^(floor(log2 amax) - 2): amax / X in [4, 8)
            assert 4.0 <= am / X < 8.0
            err = np.abs(What[i, 32 * b:32 * (b + 1)] - blk)
            # RNE on the grid: half the spacing (<= X) below 6X; saturation above
            assert np.all(err <= np.where(np.abs(blk) <= 6 * X, X, 2 * X))
    # values already on the grid times X come back exactly
    grid = mx.decode_table()[[1, 2, 3, 4, 5, 6, 7, 9, 10, 15]] * 2.0 ** -5
    row = np.concatenate([grid, np.zeros(22)]).astype(np.float32)[None, :]
    row[0, 5] = 6 * 2.0 ** -5      # amax 6 * 2^-5 -> X = 2^-5
    c, s, _ = mx.quantize(row)
    assert np.array_equal(mx.dequantize(c, s), row)


def test_packing_order_low_nibble_first():
    row = np.zeros((1, 32), dtype=np.float32)
    row[0, 0], row[0, 1], row[0, 2] = 6.0, -0.5, 1.0
    codes, scales, _ = mx.quantize(row)
    assert scales[0, 0] == 127
    assert codes[0, 0] == (0x7 | (0x9 << 4)) and codes[0, 1] == 0x2


def test_nonfinite_and_zero_blocks():
    row = np.zeros((1, 64), dtype=np.float32)
    row[0, 3] = np.nan
    row[0, 4], row[0, 5], row[0, 6] = np.inf, -2.0, 7.0
    codes, scales, flags = mx.quantize(row)
    assert scales[0, 0] == 0xFF and scales[0, 1] == 127
    assert flags == mx.FLAG_NONFINITE | mx.FLAG_ZERO_AMAX
    e = mx.unpack(codes)[0]
    assert e[3] == 0x0 and e[4] == 0x7 and e[5] == 0xC and e[6] == 0x7
    What = mx.dequantize(codes, scales)
    assert np.all(np.isnan(What[0, :32])) and np.all(What[0, 32:] == 0)
