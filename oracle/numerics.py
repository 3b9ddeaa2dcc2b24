"""Number formats used by the oracle: fp32, bf16 and OCP FP8 E4M3FN.

Everything is held in float64 numpy arrays whose values are exactly representable
in the named format; the rounding functions below are written from the formats'
definitions (round to nearest, ties to even), not from bit tricks.

E4M3FN (OCP 8-bit floating point specification): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m * 2^-9; codes
0x7F / 0xFF are NaN; there is no infinity; the largest finite magnitude is
0x7E = 1.75 * 2^8 = 448.  Block-scaled FP8 in the DeepSeek-V3 style is the format
the pages' "FP8 Training" section names for trainer GEMMs.
"""

import numpy as np

E4M3_MAX = 448.0


def _e4m3_table():
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


#: exact value of every e4m3 code (NaN for 0x7F and 0xFF)
E4M3_VALUES = _e4m3_table()
# non-negative finite codes 0..126 in ascending order of value
_POS = E4M3_VALUES[:127].copy()


def e4m3_decode(q):
    """Exact value of each code in ``q`` (uint8 array)."""
    return E4M3_VALUES[np.asarray(q, dtype=np.uint8)]


def e4m3_encode(y):
    """Round-to-nearest-even of ``y`` onto the E4M3FN grid, saturating at +-448.

    Magnitudes above 448 clamp to 448 (satfinite).  Ties go to the code with an
    even mantissa.  The sign is kept on underflow, so negative values that round
    to zero, and -0.0, give code 0x80.
    """
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    lo = np.clip(np.searchsorted(_POS, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    # codes lo and lo+1 are neighbours on the grid; exactly one of them is even
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | (neg.astype(np.uint8) << 7)


def round_binary(x, p, emin):
    """Round float64 ``x`` to a binary format with ``p`` significand bits (hidden
    bit included) and minimum normal exponent ``emin``: round to nearest, ties to
    even, gradual underflow, overflow to +-inf.  The exponent range is taken as
    fp32's (emax = 127) which bf16 shares."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| = m * 2^e with 0.5 <= m < 1
    q_exp = np.maximum(e - p, emin - (p - 1))
    quantum = np.ldexp(1.0, q_exp)
    r = np.rint(x / quantum) * quantum      # np.rint rounds half to even
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)


def f32(x):
    """Round to IEEE binary32 (numpy's float64 -> float32 cast is IEEE RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to bfloat16 (8 significand bits, fp32's exponent range), RNE."""
    return round_binary(x, 8, -126)


def bf16_bits(x):
    """uint16 bit patterns of values that are already bf16-exact."""
    v = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """float64 values of bf16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
