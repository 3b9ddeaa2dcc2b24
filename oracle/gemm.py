"""Blockwise-scaled FP8 GEMMs, accumulated in fp64.

General form, for A rows m and B rows n that share a contraction axis K split into
128-wide blocks c:
    acc[m, n] = sum_c  sA[m, c] * sB[n, c] * sum_{i<128} dec(qA[m, 128c+i]) * dec(qB[n, 128c+i])
Each inner 128-term sum is exact in fp64: every e4m3 value is an integer multiple
of 2^-9 below 2^18 units, so a product is an integer below 2^36 in units of 2^-18,
and 128 of them stay below 2^43 < 2^53.  The library keeps the same block
structure but accumulates in fp32 (MFMA accumulators rescaled once per block).

Grouped forms (rows in the expert-grouped layout of oracle.dispatch):
  * forward / dgrad:  out[r, :] = acc over K for real rows r of expert e, with B the
    expert's weight matrix given as [N, K] and its 128x128 block scales.  The
    dgrad products use the weights transposed; 128x128 blocks transpose with them.
  * wgrad:  dW[e][m, n] = acc with K running over the 128-row token blocks of the
    expert's row segment, A and B given transposed ([M, rows], [N, rows]) with one
    scale per (column, 128-row block).
"""

import numpy as np

from .numerics import e4m3_decode


def blockscaled_matmul(qa, sa, qb, sb):
    """qa [M, K] codes, sa [M, K/128]; qb [N, K] codes, sb [N, K/128] -> acc [M, N] fp64."""
    A = e4m3_decode(qa)
    B = e4m3_decode(qb)
    M, K = A.shape
    N = B.shape[0]
    assert K % 128 == 0 and B.shape[1] == K
    sa = np.asarray(sa, dtype=np.float64)
    sb = np.asarray(sb, dtype=np.float64)
    acc = np.zeros((M, N), dtype=np.float64)
    for c in range(K // 128):
        blk = slice(128 * c, 128 * c + 128)
        part = A[:, blk] @ B[:, blk].T                      # exact
        acc += (sa[:, c][:, None] * sb[:, c][None, :]) * part
    return acc


def expand_weight_scales(s_blocks):
    """128x128 block scales [N/128, K/128] -> per-row scales [N, K/128]."""
    return np.repeat(np.asarray(s_blocks, dtype=np.float64), 128, axis=0)


def grouped_forward(qa, sa, counts, offsets, qw, sw, experts=None):
    """qa [n_rows, K], sa [n_rows, K/128]; qw [L, N, K] codes, sw [L, N/128, K/128].

    Returns acc [n_rows, N] fp64 for real rows (first counts[e] rows of every
    segment); padding rows are left 0.  ``experts`` restricts the work to a subset."""
    L, N, K = qw.shape
    out = np.zeros((qa.shape[0], N), dtype=np.float64)
    for e in (range(L) if experts is None else experts):
        n = int(counts[e])
        if n == 0:
            continue
        r = slice(int(offsets[e]), int(offsets[e]) + n)
        out[r] = blockscaled_matmul(qa[r], sa[r], qw[e], expand_weight_scales(sw[e]))
    return out


def grouped_dgrad(qa, sa, counts, offsets, qw, sw, experts=None):
    """Same as grouped_forward with every expert's weight used transposed:
    qw [L, K, N] (the forward [out, in] matrix with K = out), sw [L, K/128, N/128]."""
    qwt = np.ascontiguousarray(np.swapaxes(qw, 1, 2))
    swt = np.ascontiguousarray(np.swapaxes(sw, 1, 2))
    return grouped_forward(qa, sa, counts, offsets, qwt, swt, experts)


def grouped_wgrad(qaT, saT, qbT, sbT, counts, offsets, experts=None):
    """qaT [M, n_rows] codes with scales [M, n_rows/128]; qbT [N, n_rows], [N, n_rows/128].

    dW[e] = acc over the token blocks of expert e's padded segment -> [L, M, N] fp64
    (padding rows were quantised as 0, so they add nothing)."""
    L = len(counts)
    M, N = qaT.shape[0], qbT.shape[0]
    out = np.zeros((L, M, N), dtype=np.float64)
    for e in (range(L) if experts is None else experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        cols = slice(lo, hi)
        blks = slice(lo // 128, hi // 128)
        out[e] = blockscaled_matmul(qaT[:, cols], saT[:, blks], qbT[:, cols], sbT[:, blks])
    return out
