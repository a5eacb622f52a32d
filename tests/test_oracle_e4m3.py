"""Pins for the oracle's E4M3 codec: the format's printed special values, an
independent library decode/encode, the structure of the 256-code table and
the RNE / saturation rules."""

import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import e4m3


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_format_table.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                name, bits, value = line.split()
                s, e, m = bits.split(".")
                code = (int(s, 2) << 7) | (int(e, 2) << 3) | int(m, 2)
                rows.append((name, code, float(value)))
    return rows


@pytest.mark.parametrize("name,code,value", _golden())
def test_printed_format_values(name, code, value):
    got = e4m3.decode_table()[code]
    if np.isnan(value):
        assert np.isnan(got)
    else:
        assert got == value
        assert e4m3.encode(np.float32(value)) == code
        assert e4m3.encode(np.float32(-value)) == code | 0x80


def test_decode_matches_torch_for_all_256_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_table_structure():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert pos[-1] == 448.0
    # subnormals: 8 equal steps of 2^-9 from 0
    assert np.array_equal(pos[:8], np.arange(8) * 2.0 ** -9)
    # each normal binade: 8 equal steps of 2^(e-10)
    for e in range(1, 16):
        vals = pos[8 * e: 8 * e + 8]
        if e == 15:
            vals = vals[:7]
        steps = np.diff(np.concatenate([vals, [2.0 ** (e - 6)]]))
        if e == 15:
            steps = np.diff(vals)
        assert np.all(steps == 2.0 ** (e - 10))
        assert vals[0] == 2.0 ** (e - 7)


def test_encode_decode_identity_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode_table()[codes].astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    t = e4m3.decode_table()
    for c in range(0, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2          # midpoints are exact fp32
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(mid) == even
        assert e4m3.encode(np.nextafter(mid, np.float32(np.inf))) == c + 1
        assert e4m3.encode(np.nextafter(mid, np.float32(-np.inf))) == c
        assert e4m3.encode(-mid) == even | 0x80


def test_saturation_nan_and_signed_zero():
    f = np.float32
    assert e4m3.encode(f(448.0)) == 0x7E
    assert e4m3.encode(f(455.0)) == 0x7E
    assert e4m3.encode(f(464.0)) == 0x7E
    assert e4m3.encode(f(1e30)) == 0x7E
    assert e4m3.encode(f(np.inf)) == 0x7E
    assert e4m3.encode(f(-np.inf)) == 0xFE
    assert e4m3.encode(f(-500.0)) == 0xFE
    assert e4m3.encode(f(np.nan)) == 0x7F
    assert e4m3.encode(f(0.0)) == 0x00
    assert e4m3.encode(f(-0.0)) == 0x80
    assert e4m3.encode(f(2.0 ** -10)) == 0x00          # tie with 0 -> even
    assert e4m3.encode(f(-(2.0 ** -10))) == 0x80
    assert e4m3.encode(np.nextafter(f(2.0 ** -10), f(1))) == 0x01
    assert e4m3.encode(f(1e-30)) == 0x00
    assert e4m3.encode(f(-1e-30)) == 0x80
    assert e4m3.encode(f(1e-45)) == 0x00                 # fp32 subnormal


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-14, np.log2(463.9), size=200_000))
    y = (mags * rng.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(y), ref)
