"""Pins for oracle.blockfp8: tile-by-tile brute force for every tile shape, the
saturating-code invariant, the dequantisation error bound, zero tiles, and that
row quantisation commutes with the row permutation."""

import numpy as np

from oracle import blockfp8 as Q
from oracle import dispatch as D
from oracle.numerics import E4M3_VALUES, bf16, e4m3_decode, e4m3_encode, f32
from oracle.routing import topk


def _tile(v):
    """One tile, written out scalar by scalar."""
    a = max(max(abs(float(t)) for t in v.ravel()), 2.0 ** -40)
    inv = float(np.float32(448.0 / a))
    s = float(np.float32(a / 448.0))
    q = np.array([e4m3_encode(np.array([float(np.float32(float(t) * inv))]))[0] for t in v.ravel()],
                 dtype=np.uint8).reshape(v.shape)
    return q, s


def test_1x128_brute():
    rng = np.random.default_rng(0)
    x = bf16(rng.standard_normal((3, 256)) * np.exp2(rng.integers(-20, 20, (3, 1))))
    q, s = Q.quant_1x128(x)
    for r in range(3):
        for c in range(2):
            bq, bs = _tile(x[r, 128 * c:128 * c + 128])
            assert np.array_equal(q[r, 128 * c:128 * c + 128], bq) and s[r, c] == bs


def test_128x128_brute():
    rng = np.random.default_rng(1)
    w = bf16(rng.standard_normal((2, 256, 128)) * 0.02)
    q, s = Q.quant_128x128(w)
    assert s.shape == (2, 2, 1)
    for e in range(2):
        for b in range(2):
            bq, bs = _tile(w[e, 128 * b:128 * b + 128, :])
            assert np.array_equal(q[e, 128 * b:128 * b + 128, :], bq) and s[e, b, 0] == bs


def test_128x1_t_brute_and_padding():
    rng = np.random.default_rng(2)
    src = f32(rng.standard_normal((256, 128)))
    real = np.ones(256, bool)
    real[100:128] = False                      # padding rows inside the first block
    src_garbage = src.copy()
    src_garbage[~real] = 1e6                   # padding contents must not matter
    q, s = Q.quant_128x1_t(src_garbage, real)
    assert q.shape == (128, 256) and s.shape == (128, 2)
    z = np.where(real[:, None], src, 0.0)
    for col in (0, 5, 127):
        for b in range(2):
            bq, bs = _tile(z[128 * b:128 * b + 128, col])
            assert np.array_equal(q[col, 128 * b:128 * b + 128], bq) and s[col, b] == bs
    assert np.all(q[:, 100:128] == 0)


def test_saturating_code_and_error_bound():
    rng = np.random.default_rng(3)
    x = f32(rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-30, 30, (64, 1))))
    q, s = Q.quant_1x128(x)
    qt = q.reshape(64, 8, 128)
    assert np.all(np.any((qt == 0x7E) | (qt == 0xFE), axis=2))
    deq = Q.dequant_1x128(q, s)
    # half an e4m3 ulp (2^-4 relative for normals) plus the subnormal quantum, in
    # units of the tile scale, plus fp32 rounding slack
    ss = np.repeat(s, 128, axis=1)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * ss) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)


def test_zero_and_tiny_tiles():
    x = np.zeros((2, 128))
    x[1, 3] = -0.0
    q, s = Q.quant_1x128(x)
    assert np.all(s == f32(2.0 ** -40 / 448.0))
    assert np.all(q[0] == 0) and q[1, 3] == 0x80
    t = np.zeros((1, 128))
    t[0, 0] = 2.0 ** -60
    q, s = Q.quant_1x128(t)
    assert np.all(q == 0)


def test_quant_commutes_with_permutation():
    rng = np.random.default_rng(4)
    T, E, k, d = 80, 16, 4, 256
    ids, _ = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    x = bf16(rng.standard_normal((T, d)))
    c, o, rp, pr = D.permute_index(ids, 4, 8)
    q1, s1 = Q.quant_1x128(D.gather_rows(x, rp, k))
    qx, sx = Q.quant_1x128(x)
    real = rp >= 0
    assert np.array_equal(q1[real], qx[rp[real] // k]) and np.array_equal(s1[real], sx[rp[real] // k])


def test_decode_closed_form_in_quant_context():
    # one tile whose amax is 448 exactly quantises with scale 1 and returns the grid
    v = E4M3_VALUES[:127].copy()
    v = np.concatenate([v, [0.0]])[None, :]
    q, s = Q.quant_1x128(v)
    assert s[0, 0] == 1.0 and np.array_equal(e4m3_decode(q), v)
