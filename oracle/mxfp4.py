"""OCP MX FP4 (MXFP4) codec (oracle; test infrastructure only).

Definitions restated from the OCP Microscaling Formats (MX) Specification,
version 1.0 (the FP4 E2M1 element format, the E8M0 scale format and the
MXFP4 block of 32 elements):

* E2M1 element: one sign bit, two exponent bits with bias 1, one mantissa
  bit.  Exponent field 0 encodes the subnormal m * 0.5; the magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6.  There is no infinity and no NaN.
* E8M0 scale: eight exponent bits with bias 127, no sign and no mantissa;
  code c stands for 2^(c - 127), code 0xFF for NaN.
* A block of 32 consecutive elements shares one scale X = 2^e with
  e = floor(log2(amax)) - emax, emax = 2 being the exponent of the largest
  E2M1 normal (6 = 1.5 * 2^2); element i is stored as E2M1(v_i / X).

The GIFT review names FP4 only as the direction where the method should
gain more ("Core claim" and the abstract's lower bit-widths); the choices
below are this implementation's reading where the specification leaves
room:

* encode rounds v / X to the nearest E2M1 value with ties to the even code
  (code LSB 0), saturates magnitudes above 6 (and +-inf) to +-6, keeps the
  sign of zero and of values that round to zero (-0 -> 0x8), and maps NaN
  to code 0 (+0);
* e is clamped to the E8M0 range [-127, 127]; an all-zero block gets X = 1
  (code 127) and raises FLAG_ZERO_AMAX; a block whose amax is NaN or +inf
  gets the NaN scale (code 0xFF), decodes to NaN, and raises FLAG_NONFINITE;
  its elements are encoded with X = 1;
* amax is the largest |v| bit pattern, as for E4M3 (NaN > +inf > finite);
* two elements per byte, the lower-indexed one in the low nibble; a d_out x
  d_in tensor (d_in % 32 == 0) has d_out x d_in/2 code bytes and
  d_out x d_in/32 scale bytes, both row-major.

All arithmetic is exact: v / X is a power-of-two scaling of an fp32 value,
and every E2M1 value, midpoint and decoded value is representable.
"""

import numpy as np

BLOCK = 32
EMAX_ELEM = 2
SCALE_BIAS = 127
SCALE_NAN = 0xFF
MAX_ELEM = 6.0
FLAG_NONFINITE = 1
FLAG_ZERO_AMAX = 2

# magnitudes of the codes 0..7 (code 8..15: the same, negative)
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def decode_table():
    """fp64 value of each of the 16 E2M1 codes."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp_field = (code >> 1) & 0x3
        mant = code & 0x1
        if exp_field == 0:
            vals[code] = sign * mant * 0.5
        else:
            vals[code] = sign * (1.0 + mant / 2.0) * 2.0 ** (exp_field - 1)
    return vals


_TABLE = decode_table()


def encode_elements(y):
    """fp32 array (already divided by the block scale) -> E2M1 codes 0..15
    (uint8, one per element): RNE, saturating, see the module doc."""
    y = np.asarray(y, dtype=np.float32)
    y64 = y.astype(np.float64)
    isnan = np.isnan(y64)
    neg = np.signbit(y) & ~isnan
    mag = np.where(isnan, 0.0, np.minimum(np.abs(y64), MAX_ELEM))
    lo = np.clip(np.searchsorted(_MAG, mag, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = mag - _MAG[lo]
    d_hi = _MAG[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(neg, code | np.uint8(0x8), code).astype(np.uint8)


def decode_elements(codes):
    """E2M1 codes (uint8 0..15) -> fp64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def scale_exponent(amax):
    """(E8M0 code, flags) for a block amax given as fp32."""
    a = np.float32(amax)
    if np.isnan(a) or np.isinf(a):
        return SCALE_NAN, FLAG_NONFINITE
    if a == 0:
        return SCALE_BIAS, FLAG_ZERO_AMAX
    bits = int(np.array([a], dtype=np.float32).view(np.uint32)[0]) & 0x7FFFFFFF
    field = bits >> 23
    if field:
        floor_log2 = field - 127
    else:  # subnormal amax: position of the leading mantissa bit
        floor_log2 = -149 + (bits.bit_length() - 1)
    e = min(max(floor_log2 - EMAX_ELEM, -127), 127)
    return e + SCALE_BIAS, 0


def scale_value(code):
    """fp64 value of an E8M0 code (NaN for 0xFF)."""
    code = int(code)
    return float("nan") if code == SCALE_NAN else 2.0 ** (code - SCALE_BIAS)


def amax(block32):
    """max |v| as the largest |v| bit pattern, returned as fp32."""
    b = np.ascontiguousarray(block32, dtype=np.float32)
    bits = b.view(np.uint32) & np.uint32(0x7FFFFFFF)
    return np.array([bits.max()], dtype=np.uint32).view(np.float32)[0]


def quantize(w32):
    """d_out x d_in fp32 (d_in % 32 == 0) -> (codes d_out x d_in/2 uint8,
    scales d_out x d_in/32 uint8 E8M0, flags)."""
    w32 = np.asarray(w32, dtype=np.float32)
    d_out, d_in = w32.shape
    if d_in % BLOCK:
        raise ValueError("MXFP4 needs d_in % 32 == 0")
    nb = d_in // BLOCK
    elems = np.empty((d_out, d_in), dtype=np.uint8)
    scales = np.empty((d_out, nb), dtype=np.uint8)
    flags = 0
    for i in range(d_out):
        for b in range(nb):
            blk = w32[i, b * BLOCK:(b + 1) * BLOCK]
            code, f = scale_exponent(amax(blk))
            flags |= f
            scales[i, b] = code
            e = 0 if code == SCALE_NAN else code - SCALE_BIAS
            # v / 2^e: exact in fp64, then the fp32 value the device forms
            y = (blk.astype(np.float64) * 2.0 ** (-e)).astype(np.float32)
            elems[i, b * BLOCK:(b + 1) * BLOCK] = encode_elements(y)
    codes = (elems[:, 0::2] | (elems[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales, flags


def unpack(codes):
    """d_out x d_in/2 bytes -> d_out x d_in E2M1 codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequantize(codes, scales):
    """(codes, scales) -> fp32 d_out x d_in: E2M1 value * X (exact)."""
    vals = decode_elements(unpack(codes))
    sc = np.array([[scale_value(c) for c in row] for row in np.asarray(scales)], dtype=np.float64)
    return (vals * np.repeat(sc, BLOCK, axis=1)).astype(np.float32)
