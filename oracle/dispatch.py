"""Dispatch and combine on one GPU's share of experts.

The pages ("RL at 1T scale", sections "Wide Expert Parallelism" and "Parallelism
strategies / Expert Parallel") place each GPU's experts between a per-layer
dispatch and a per-layer combine.  On one GPU the dispatch is a local
permutation: every (token, slot) pair whose expert lies in [e0, e0 + L) is moved
exactly once into a row block owned by that expert; no capacity, no dropping.

Permutation index (plain definition = stable sort):
  * pair p = t*k + j is local iff e0 <= ids[t, j] < e0 + L; le = ids - e0
  * counts[e]    = number of local pairs with le = e
  * offsets[0]   = 0, offsets[e+1] = offsets[e] + ceil(counts[e] / 128) * 128
  * the pairs of expert e, in ascending p, occupy rows offsets[e], offsets[e]+1, ...
  * row_pair[r]  = p for a real row, -1 for a padding row (r < offsets[L])
  * pair_row[p]  = r for a local pair, -1 otherwise

Combine:  y[t] = bf16( sum over local j, ascending, of w[t, j] * Y[pair_row[t, j]] ),
summed in fp64; a token with no local pair gets +0.
"""

import numpy as np

from .numerics import bf16

ALIGN = 128


def permute_index(ids, e0, L, align=ALIGN):
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    le = (ids - e0).ravel()
    local = (le >= 0) & (le < L)
    pairs = np.flatnonzero(local)                   # ascending pair index
    lep = le[pairs]
    order = np.argsort(lep, kind="stable")          # by expert, ties by pair index
    counts = np.bincount(lep, minlength=L).astype(np.int32)
    padded = (counts.astype(np.int64) + align - 1) // align * align
    offsets = np.zeros(L + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    n_rows = int(offsets[L])
    row_pair = np.full(n_rows, -1, dtype=np.int32)
    pair_row = np.full(T * k, -1, dtype=np.int32)
    starts = np.zeros(L + 1, dtype=np.int64)
    starts[1:] = np.cumsum(counts)
    sorted_pairs = pairs[order]
    sorted_le = lep[order]
    rank = np.arange(len(sorted_pairs)) - starts[sorted_le]
    rows = offsets[sorted_le] + rank
    row_pair[rows] = sorted_pairs
    pair_row[sorted_pairs] = rows
    return counts, offsets.astype(np.int32), row_pair, pair_row.reshape(T, k)


def real_rows(row_pair):
    return np.asarray(row_pair) >= 0


def gather_rows(x, row_pair, k):
    """X_perm[r] = x[row_pair[r] // k] for real rows, +0 for padding rows."""
    x = np.asarray(x, dtype=np.float64)
    rp = np.asarray(row_pair)
    out = np.zeros((len(rp), x.shape[1]), dtype=np.float64)
    real = rp >= 0
    out[real] = x[rp[real] // k]
    return out


def combine(Y, pair_row, w):
    """Y [n_rows, d] values, pair_row [T, k], w [T, k] (None means weights of 1,
    the plain unpermute-sum used for the input gradient).  Returns bf16-valued y."""
    Y = np.asarray(Y, dtype=np.float64)
    pair_row = np.asarray(pair_row)
    T, k = pair_row.shape
    y = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):                               # ascending slot order
        r = pair_row[:, j]
        m = r >= 0
        wj = 1.0 if w is None else np.asarray(w, dtype=np.float64)[m, j][:, None]
        y[m] += wj * Y[r[m]]
    return bf16(y)
