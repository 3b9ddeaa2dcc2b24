"""Block-scaled FP8 e4m3 quantisation (the DeepSeek-V3 scheme that the pages'
"FP8 Training" section says the trainer uses for its GEMMs).

For every tile of source values v (each value exactly representable in fp32):
    a   = max(max|v|, 2^-40)
    inv = f32(448 / a)          correctly rounded fp32 division
    s   = f32(a / 448)          the tile's fp32 scale, stored
    q   = e4m3(f32(v * inv))    one fp32 multiply, then RNE-satfinite to e4m3
and the dequantised value is dec(q) * s.

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


def _quant_tiles(v, axis):
    """Quantise ``v`` with one tile per slice along ``axis`` of a tiled view."""
    a = np.maximum(np.max(np.abs(v), axis=axis, keepdims=True), EPS)
    inv = f32(E4M3_MAX / a)
    s = f32(a / E4M3_MAX)
    q = e4m3_encode(f32(v * inv))
    return q, np.squeeze(s, axis=axis)


def quant_1x128(src):
    """src [rows, cols] (cols % 128 == 0) -> q uint8 [rows, cols], s [rows, cols/128]."""
    src = np.asarray(src, dtype=np.float64)
    rows, cols = src.shape
    assert cols % 128 == 0
    q, s = _quant_tiles(src.reshape(rows, cols // 128, 128), axis=2)
    return q.reshape(rows, cols), s


def quant_128x128(w):
    """w [L, out, in] (out, in % 128 == 0) -> q uint8 [L, out, in], s [L, out/128, in/128]."""
    w = np.asarray(w, dtype=np.float64)
    L, n_out, n_in = w.shape
    assert n_out % 128 == 0 and n_in % 128 == 0
    t = w.reshape(L, n_out // 128, 128, n_in // 128, 128).transpose(0, 1, 3, 2, 4)
    t = t.reshape(L, n_out // 128, n_in // 128, 128 * 128)
    q, s = _quant_tiles(t, axis=3)
    q = q.reshape(L, n_out // 128, n_in // 128, 128, 128).transpose(0, 1, 3, 2, 4)
    return q.reshape(L, n_out, n_in), s


def quant_128x1_t(src, real_row):
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
    q, s = _quant_tiles(t, axis=2)
    return q.reshape(cols, n_rows), s


def dequant_1x128(q, s):
    from .numerics import e4m3_decode
    rows, cols = q.shape
    return (e4m3_decode(q).reshape(rows, cols // 128, 128) * s[:, :, None]).reshape(rows, cols)


def dequant_128x128(q, s):
    from .numerics import e4m3_decode
    return e4m3_decode(q) * np.repeat(np.repeat(s, 128, axis=1), 128, axis=2)
