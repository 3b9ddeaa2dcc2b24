"""Block-scaled FP8 e4m3 quantisation (the DeepSeek-V3 scheme that the pages'
"FP8 Training" section says the trainer uses for its GEMMs).

For every tile of source values v (each value exactly representable in fp32):
    a   = max(max|v|, 2^-40)
    inv = f32(448 / a)          correctly rounded fp32 division
    s   = f32(a / 448)          the tile's fp32 scale, stored
    q   = e4m3(f32(v * inv))    one fp32 multiply, then RNE-satfinite to e4m3
and the dequantised value is dec(q) * s.

Power-of-two variant (pow2=True; the UE8M0 scales that gfx950's block-scaled
MFMA applies in hardware, a variant of the same block scaling): the scale is
the smallest power of two that brings the tile into range,
    e   = min { integer e : a <= 448 * 2^e }
    s   = 2^e,  inv = 2^-e      (both exact)
    q   = e4m3(v * 2^-e)        (the product is exact; one RNE-satfinite rounding)
so a / s lies in (224, 448].

f32(448 / a) is computed as an fp64 quotient rounded once more to fp32; for
division of fp32 operands this double rounding equals a single correct rounding
because binary64 carries more than 2*24 + 2 significand bits.

Tile shapes:
  * 1x128   along a row (the consuming GEMM's K axis);        scales [rows, cols/128]
  * 128x128 weight blocks of [out, in] per expert;             scales [L, out/128, in/128]
  * 128x1   along rows, over the expert-grouped row layout whose segments start at
            multiples of 128 rows, so every 128-row block lies inside one expert;
            rows that are padding count as 0.  Output is transposed:
            q [cols, n_rows], scales [cols, n_rows/128].
"""

import numpy as np

from .numerics import E4M3_MAX, e4m3_encode, f32

EPS = 2.0 ** -40


def pow2_exponent(a):
    """min { integer e : a <= 448 * 2^e } for a > 0, elementwise.

    With a = m * 2^E (frexp, m in [0.5, 1)) and 448 = 0.875 * 2^9: e = E - 9
    when m <= 0.875, else E - 8 (exact: frexp and the comparison are exact)."""
    m, E = np.frexp(np.asarray(a, dtype=np.float64))
    return np.where(m <= 0.875, E - 9, E - 8).astype(np.int64)


def _quant_tiles(v, axis, pow2=False):
    """Quantise ``v`` with one tile per slice along ``axis`` of a tiled view."""
    a = np.maximum(np.max(np.abs(v), axis=axis, keepdims=True), EPS)
    if pow2:
        e = pow2_exponent(a)
        s = np.ldexp(1.0, e)
        q = e4m3_encode(np.ldexp(v, -e))
    else:
        inv = f32(E4M3_MAX / a)
        s = f32(a / E4M3_MAX)
        q = e4m3_encode(f32(v * inv))
    return q, np.squeeze(s, axis=axis)


def quant_1x128(src, pow2=False):
    """src [rows, cols] (cols % 128 == 0) -> q uint8 [rows, cols], s [rows, cols/128]."""
    src = np.asarray(src, dtype=np.float64)
    rows, cols = src.shape
    assert cols % 128 == 0
    q, s = _quant_tiles(src.reshape(rows, cols // 128, 128), axis=2, pow2=pow2)
    return q.reshape(rows, cols), s


def quant_128x128(w, pow2=False):
    """w [L, out, in] (out, in % 128 == 0) -> q uint8 [L, out, in], s [L, out/128, in/128]."""
    w = np.asarray(w, dtype=np.float64)
    L, n_out, n_in = w.shape
    assert n_out % 128 == 0 and n_in % 128 == 0
    t = w.reshape(L, n_out // 128, 128, n_in // 128, 128).transpose(0, 1, 3, 2, 4)
    t = t.reshape(L, n_out // 128, n_in // 128, 128 * 128)
    q, s = _quant_tiles(t, axis=3, pow2=pow2)
    q = q.reshape(L, n_out // 128, n_in // 128, 128, 128).transpose(0, 1, 3, 2, 4)
    return q.reshape(L, n_out, n_in), s


def quant_128x1_t(src, real_row, pow2=False):
    """Quantise along rows in 128-row blocks and return the transposed result.

    src      [n_rows, cols], n_rows % 128 == 0, rows in expert-grouped order whose
             expert segments start at multiples of 128
    real_row bool [n_rows]; False rows are padding and are quantised as 0
    returns  q uint8 [cols, n_rows], s [cols, n_rows/128]
    """
    src = np.where(np.asarray(real_row)[:, None], np.asarray(src, dtype=np.float64), 0.0)
    n_rows, cols = src.shape
    assert n_rows % 128 == 0
    t = src.T.reshape(cols, n_rows // 128, 128)
    q, s = _quant_tiles(t, axis=2, pow2=pow2)
    return q.reshape(cols, n_rows), s


def dequant_1x128(q, s):
    from .numerics import e4m3_decode
    rows, cols = q.shape
    return (e4m3_decode(q).reshape(rows, cols // 128, 128) * s[:, :, None]).reshape(rows, cols)


def dequant_128x128(q, s):
    from .numerics import e4m3_decode
    return e4m3_decode(q) * np.repeat(np.repeat(s, 128, axis=1), 128, axis=2)
