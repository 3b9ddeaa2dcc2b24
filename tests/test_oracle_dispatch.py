"""Pins for oracle.dispatch: the permutation index against a brute-force loop and
its invariants (every local pair dispatched exactly once, counts, 128-aligned
offsets, ascending tokens within an expert), and the combine's closed forms."""

import numpy as np

from oracle import dispatch as D
from oracle.numerics import bf16
from oracle.routing import topk


def _brute(ids, e0, L):
    T, k = ids.shape
    rows_of = {e: [] for e in range(L)}
    for t in range(T):
        for j in range(k):
            le = int(ids[t, j]) - e0
            if 0 <= le < L:
                rows_of[le].append(t * k + j)
    counts = [len(rows_of[e]) for e in range(L)]
    offsets = [0]
    for e in range(L):
        offsets.append(offsets[-1] + -(-counts[e] // 128) * 128)
    row_pair = [-1] * offsets[-1]
    pair_row = [-1] * (T * k)
    for e in range(L):
        for i, p in enumerate(rows_of[e]):
            row_pair[offsets[e] + i] = p
            pair_row[p] = offsets[e] + i
    return counts, offsets, row_pair, pair_row


def test_permute_brute_force():
    rng = np.random.default_rng(0)
    for T, E, k, e0, L in [(100, 8, 2, 0, 8), (300, 64, 6, 16, 8), (50, 16, 4, 12, 4),
                           (1, 8, 8, 0, 8), (260, 4, 1, 0, 4)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = topk(lg, k)
        c, o, rp, pr = D.permute_index(ids, e0, L)
        bc, bo, brp, bpr = _brute(ids, e0, L)
        assert list(c) == bc and list(o) == bo and list(rp) == brp and list(pr.ravel()) == bpr


def test_permute_invariants():
    rng = np.random.default_rng(1)
    T, E, k, e0, L = 2000, 256, 8, 32, 32
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = topk(lg, k)
    c, o, rp, pr = D.permute_index(ids, e0, L)
    local = ((ids >= e0) & (ids < e0 + L)).ravel()
    P = int(local.sum())
    assert c.sum() == P
    assert np.all(o % 128 == 0) and o[0] == 0 and np.all(np.diff(o) >= c)
    real = np.flatnonzero(rp >= 0)
    assert len(real) == P
    # bijection between real rows and local pairs
    assert np.array_equal(np.sort(rp[real]), np.flatnonzero(local))
    assert np.all(pr.ravel()[rp[real]] == real)
    assert np.all(pr.ravel()[~local] == -1)
    for e in range(L):
        seg = rp[o[e]:o[e] + c[e]]
        assert np.all(ids.ravel()[seg] == e0 + e)
        assert np.all(np.diff(seg // k) > 0)
        assert np.all(rp[o[e] + c[e]:o[e + 1]] == -1)


def test_permute_all_local_sums_to_Tk_and_skew():
    ids = np.zeros((300, 1), dtype=np.int32)                 # every token to expert 0
    c, o, rp, pr = D.permute_index(ids, 0, 4)
    assert list(c) == [300, 0, 0, 0] and list(o) == [0, 384, 384, 384, 384]
    assert np.array_equal(rp[:300], np.arange(300)) and np.all(rp[300:] == -1)
    ids = np.array([[3, 1], [1, 3], [0, 2]], dtype=np.int32)
    c, o, rp, pr = D.permute_index(ids, 0, 4)
    assert c.sum() == 6


def test_combine_closed_forms():
    rng = np.random.default_rng(2)
    T, E, k, d = 64, 8, 3, 256
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = topk(lg, k)
    x = bf16(rng.standard_normal((T, d)))
    c, o, rp, pr = D.permute_index(ids, 0, E)
    Y = D.gather_rows(x, rp, k)                  # every row holds its token's x
    # sum_j w_j x = x (1 + O(1e-7)), which rounds back to x in bf16
    assert np.array_equal(D.combine(Y, pr, w), x)
    # weights off: sum of k copies, exact in bf16 for k = 2 and x * 3 rounded once
    assert np.array_equal(D.combine(Y, pr, None), bf16(3.0 * x))
    ids1, w1 = topk(lg, 1)
    c, o, rp, pr = D.permute_index(ids1, 0, E)
    Y1 = bf16(rng.standard_normal((len(rp), d)))
    y1 = D.combine(Y1, pr, w1)
    assert np.array_equal(y1, Y1[pr[:, 0]])


def test_combine_nonlocal_tokens_zero():
    ids = np.array([[5, 6], [0, 7], [1, 2]], dtype=np.int32)
    w = np.full((3, 2), 0.5)
    c, o, rp, pr = D.permute_index(ids, 0, 4)
    Y = np.ones((len(rp), 128))
    y = D.combine(Y, pr, w)
    assert np.all(y[0] == 0) and not np.any(np.signbit(y[0]))
    assert np.all(y[1] == 0.5) and np.all(y[2] == 1.0)
