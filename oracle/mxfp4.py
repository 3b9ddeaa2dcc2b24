"""MXFP4 expert weights: 4-bit E2M1 elements with one power-of-two (E8M0) scale
per block of 32 consecutive values along the contraction axis.

Test infrastructure only: nothing on the product path imports this module.

Why this format: the pages name 4-bit (NVFP4) training and inference as future
work ("RL at 1T scale", section on future work).  The 4-bit block format that
gfx950's block-scaled matrix instruction applies natively is the OCP
Microscaling (MX) FP4 format, so the expert weights take that form here; the
activations stay block-scaled FP8 with power-of-two 1x128 scales.

Definitions (OCP Microscaling Formats specification v1.0: the E2M1 element
format and the conversion of a vector of scalars to an MX block):

E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa bit.  Codes 0..7 are the
magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.  No inf or NaN.

One block V of 32 values:
    E = floor(log2(max|V|)) - 2     (2 is the exponent of E2M1's largest
                                     normal, 6 = 1.5 * 2^2), clamped to
                                     [-127, 127]; an all-zero block takes -127
    X = 2^E                          stored as the E8M0 code E + 127
    P_i = e2m1(V_i / X)              nearest magnitude, ties to the even code,
                                     magnitudes above 6 clamp to 6, sign kept
                                     (so -0 and small negatives give code 8)
    decoded value  dec(P_i) * X
so max|V| / X lies in [4, 8): a block's largest values may saturate to 6 X.

Packing of a row: element 2b in the low nibble of byte b, element 2b + 1 in
the high nibble.  A weight matrix [N, K] (rows = output features) becomes
codes [N, K/2] bytes and scales [N, K/32] E8M0 bytes.
"""

import numpy as np

from .numerics import e4m3_decode

BLOCK = 32
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
EMAX_ELEM = 2


def e2m1_decode(c):
    """Value of each 4-bit code (array of ints 0..15)."""
    c = np.asarray(c, dtype=np.int64)
    v = E2M1_MAG[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(y):
    """Nearest E2M1 code of each value, ties to the even code (the code whose
    mantissa bit is 0), magnitudes above 6 clamped to 6, sign kept."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E2M1_MAX)
    lo = np.clip(np.searchsorted(E2M1_MAG, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_MAG[lo]
    d_hi = E2M1_MAG[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo)
    return (code | (neg.astype(np.int64) << 3)).astype(np.uint8)


def shared_exponent(amax):
    """E = floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)            # amax = m * 2^k, m in [0.5, 1): floor(log2) = k - 1
    e = np.where(amax > 0, k - 1 - EMAX_ELEM, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quant_mx(w):
    """MXFP4 of w [..., K] along the last axis (K % 32 == 0).

    Returns (codes [..., K] uint8 in 0..15, unpacked; scale codes [..., K/32]
    uint8 = E + 127)."""
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[-1]
    assert K % BLOCK == 0
    blk = w.reshape(w.shape[:-1] + (K // BLOCK, BLOCK))
    E = shared_exponent(np.max(np.abs(blk), axis=-1))
    codes = e2m1_encode(np.ldexp(blk, -E[..., None]))
    return codes.reshape(w.shape), (E + 127).astype(np.uint8)


def dequant_mx(codes, scales):
    """Values of unpacked codes [..., K] with E8M0 scale codes [..., K/32]."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    v = e2m1_decode(codes).reshape(codes.shape[:-1] + (K // BLOCK, BLOCK))
    E = np.asarray(scales, dtype=np.int64) - 127
    return np.ldexp(v, E[..., None]).reshape(codes.shape)


def pack(codes):
    """[..., K] codes -> [..., K/2] bytes, element 2b in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """[..., K/2] bytes -> [..., K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def matmul(qa, sa, codes_b, scales_b):
    """FP8 activations times MXFP4 weights, in fp64.

    qa [M, K] e4m3 codes with 1x128 scales sa [M, K/128]; codes_b [N, K]
    unpacked E2M1 codes with scales_b [N, K/32] (E8M0 codes).
        acc[m, n] = sum_k sa[m, k/128] dec8(qa[m, k]) * 2^(eb[n, k/32] - 127) dec4(b[n, k])
    Every product is exact in fp64 and the sum is taken in fp64."""
    A = e4m3_decode(qa) * np.repeat(np.asarray(sa, dtype=np.float64), 128, axis=1)
    B = dequant_mx(codes_b, scales_b)
    return A @ B.T


def grouped_forward(qa, sa, counts, offsets, codes_w, scales_w, experts=None):
    """Per-expert matmul over the expert-grouped rows: qa [n_rows, K], sa
    [n_rows, K/128]; codes_w [L, N, K] unpacked, scales_w [L, N, K/32].
    Real rows get acc; padding rows stay 0."""
    L, N, K = codes_w.shape
    out = np.zeros((qa.shape[0], N))
    for e in (range(L) if experts is None else experts):
        n = int(counts[e])
        if n:
            r = slice(int(offsets[e]), int(offsets[e]) + n)
            out[r] = matmul(qa[r], sa[r], codes_w[e], scales_w[e])
    return out
