"""OCP FP8 E4M3 codec (oracle; test infrastructure only).

Definition restated from "FP8 formats" (reference [28] of the GIFT review;
the E4M3 row of its format table): one sign bit, four exponent bits with
bias 7, three mantissa bits.  Exponent field 0 encodes subnormals
m/8 * 2^-6; S.1111.111 is the only NaN pattern (0x7F, 0xFF); there is no
infinity, so the largest finite magnitude is S.1111.110 = 1.75 * 2^8 = 448.

The GIFT review only says "FP8" (sections "The pith" and the abstract); the
E4M3 choice and the conversion rules below are this implementation's
reading:

* encode takes an fp32 value, rounds to the nearest E4M3 value with ties to
  the even code (code LSB 0), saturates every magnitude above 448 (and
  +-inf) to +-448, keeps the sign of zero and of values that round to zero
  (-0 -> 0x80), and maps NaN to 0x7F;
* decode is exact (every E4M3 value is an fp32 and an fp64 value).

All arithmetic here is exact: fp32 inputs, E4M3 values and their midpoints
are all fp64-representable, so the nearest-value search below makes no
rounding decision of its own.
"""

import numpy as np

EXP_BIAS = 7
MAX_FINITE = 448.0
NAN_CODE = 0x7F
MAX_CODE = 0x7E          # +448
NUM_CODES = 256


def decode_table():
    """fp64 value of each of the 256 codes (NaN at 0x7F and 0xFF)."""
    vals = np.empty(NUM_CODES, dtype=np.float64)
    for code in range(NUM_CODES):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            vals[code] = np.nan
        elif exp_field == 0:
            vals[code] = sign * (mant / 8.0) * 2.0 ** (1 - EXP_BIAS)
        else:
            vals[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - EXP_BIAS)
    return vals


_TABLE = decode_table()
# codes 0x00..0x7E in increasing order of value: 0, 2^-9, ..., 448
_POS = _TABLE[:MAX_CODE + 1].copy()


def decode(codes):
    """codes (uint8 array) -> fp32 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes].astype(np.float32)


def encode(y):
    """fp32 array -> uint8 E4M3 codes (RNE, saturating, see module doc)."""
    y = np.asarray(y, dtype=np.float32)
    y64 = y.astype(np.float64)
    neg = np.signbit(y)
    mag = np.abs(y64)
    isnan = np.isnan(y64)
    mag = np.where(isnan, 0.0, np.minimum(mag, MAX_FINITE))
    # _POS[lo] <= mag <= _POS[lo + 1]
    lo = np.searchsorted(_POS, mag, side="right") - 1
    lo = np.clip(lo, 0, MAX_CODE)
    hi = np.minimum(lo + 1, MAX_CODE)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    mcode = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(neg, mcode | np.uint8(0x80), mcode).astype(np.uint8)
    return np.where(isnan, np.uint8(NAN_CODE), code).astype(np.uint8)
