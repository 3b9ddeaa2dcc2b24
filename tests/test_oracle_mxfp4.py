"""Pins for oracle.mxfp4 (MXFP4 weights: E2M1 codes, E8M0 scale per 32 values):
the code table against the OCP MX specification's points, rounding against a
brute-force nearest search, the shared exponent against a search over
integers, special blocks, the nibble packing, the GEMM against scalar loops, and
the MXFP4 forward chain against the FP8 chain on weights both represent exactly."""

import os

import numpy as np

from oracle import blockfp8 as Q
from oracle import layer as OL
from oracle import mxfp4 as MX
from oracle.numerics import bf16, e4m3_decode
from oracle.routing import topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_spec_points.txt")


def test_decode_matches_spec_points():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        c = int(code, 16)
        got = MX.e2m1_decode(np.array([c]))[0]
        assert got == float(val) and np.signbit(got) == val.startswith("-"), code


def _brute_code(y):
    """Nearest of the 8 magnitudes by trying each; a tie takes the even code."""
    a = abs(y)
    best, bestd = None, None
    for c in range(8):
        d = abs(a - MX.E2M1_MAG[c])
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (8 if np.signbit(y) else 0)


def test_encode_brute_force():
    rng = np.random.default_rng(1)
    mags = MX.E2M1_MAG
    mids = (mags[1:] + mags[:-1]) / 2
    special = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 10), [6.5, 7.99, 100.0, 1e-30]])
    y = np.concatenate([special, -special, rng.uniform(-8, 8, 4000), [0.0, -0.0]])
    got = MX.e2m1_encode(y)
    for v, c in zip(y, got):
        assert c == _brute_code(float(v)), v
    # every code survives a decode / encode round trip
    codes = np.arange(16)
    assert np.array_equal(MX.e2m1_encode(MX.e2m1_decode(codes)), codes)


def _brute_exponent(amax):
    if amax == 0:
        return -127
    for e in range(-200, 200):
        if 4.0 <= amax / 2.0 ** e < 8.0:
            return max(-127, min(127, e))
    raise AssertionError(amax)


def test_shared_exponent_brute_force():
    rng = np.random.default_rng(2)
    a = np.exp2(rng.uniform(-140, 120, 400))
    edges = [f * 2.0 ** k for k in range(-130, 120, 9) for f in (4.0, 6.0, 8.0, np.nextafter(8.0, 0), 5.0)]
    a = np.concatenate([a, edges, [0.0, 2.0 ** -149, 2.0 ** -126]])
    for v, e in zip(a, MX.shared_exponent(a)):
        assert e == _brute_exponent(float(v)), v


def test_blocks_codes_range_and_error():
    rng = np.random.default_rng(3)
    w = bf16(rng.standard_normal((37, 256)) * np.exp2(rng.integers(-20, 20, (37, 1))))
    codes, sc = MX.quant_mx(w)
    assert codes.shape == w.shape and sc.shape == (37, 8)
    deq = MX.dequant_mx(codes, sc)
    for r in range(37):
        for b in range(8):
            v = w[r, 32 * b:32 * b + 32]
            X = 2.0 ** (int(sc[r, b]) - 127)
            assert 4.0 <= np.max(np.abs(v)) / X < 8.0
            for i in range(32):
                assert codes[r, 32 * b + i] == _brute_code(v[i] / X)
            # error: half the local grid spacing, or the saturation excess above 6 X
            a = np.abs(v) / X
            half = np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))
            bound = np.where(a > 6.0, a - 6.0, half) * X
            assert np.all(np.abs(deq[r, 32 * b:32 * b + 32] - v) <= bound)


def test_special_blocks():
    z = np.zeros((1, 32))
    c, s = MX.quant_mx(z)
    assert np.all(c == 0) and s[0, 0] == 0
    for k in (-20, 0, 13):
        v = np.full((1, 32), 0.5 * 2.0 ** k)
        v[0, 5] = 6.0 * 2.0 ** k                   # amax = 6 * 2^k: X = 2^k, exact
        c, s = MX.quant_mx(v)
        assert s[0, 0] == k + 127 and c[0, 5] == 7 and np.all(MX.dequant_mx(c, s) == v)
        v[0, 5] = -7.5 * 2.0 ** k                  # saturates to -6 * 2^k
        c, s = MX.quant_mx(v)
        assert s[0, 0] == k + 127 and c[0, 5] == 15
        assert MX.dequant_mx(c, s)[0, 5] == -6.0 * 2.0 ** k
    c, _ = MX.quant_mx(np.array([[-0.0] + [1.0] * 31]))
    assert c[0, 0] == 8                            # sign kept on zero


def test_pack_nibble_order():
    codes = np.array([[2, 15, 0, 7]], dtype=np.uint8)      # 1.0, -6.0, 0, 6.0
    p = MX.pack(codes)
    assert p.tolist() == [[0xF2, 0x70]]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(MX.unpack(MX.pack(c)), c)


def test_matmul_scalar_loops():
    rng = np.random.default_rng(5)
    M, N, K = 3, 2, 256
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38                     # no NaN codes
    sa = np.exp2(rng.integers(-5, 5, (M, K // 128))).astype(np.float64)
    cb = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sb = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    got = MX.matmul(qa, sa, cb, sb)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                a = float(e4m3_decode(np.array([qa[m, k]]))[0]) * sa[m, k // 128]
                b = float(MX.E2M1_MAG[cb[n, k] & 7]) * (-1.0 if cb[n, k] & 8 else 1.0) * 2.0 ** (int(sb[n, k // 32]) - 127)
                acc += a * b
            assert got[m, n] == acc


def test_forward_chain_matches_fp8_on_shared_grid():
    """Weights whose every 32-block has amax 6 * 2^k with one k per 128x128
    tile are represented exactly both ways (E2M1 values are e4m3 values), so
    the MXFP4 chain and the power-of-two FP8 chain compute the same numbers."""
    rng = np.random.default_rng(6)
    T, d, f, E, L, k = 64, 256, 128, 8, 8, 2

    def grid_weights(rows, cols):
        mag = MX.E2M1_MAG[rng.integers(0, 8, (L, rows, cols))]
        sign = np.where(rng.random((L, rows, cols)) < 0.5, -1.0, 1.0)
        w = mag * sign
        w[:, :, ::32] = 6.0                                        # amax 6 in every 32-block
        kexp = rng.integers(-9, -5, (L, rows // 128, cols // 128))
        return w * np.exp2(np.repeat(np.repeat(kexp, 128, axis=1), 128, axis=2))

    W13, W2 = grid_weights(2 * f, d), grid_weights(d, f)
    x = bf16(rng.standard_normal((T, d)))
    ids, w = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    wmx = OL.quantize_weights(W13, W2, mx=True)
    wp2 = OL.quantize_weights(W13, W2, pow2=True)
    assert np.array_equal(MX.dequant_mx(*wmx[0][:2]), W13)
    assert np.array_equal(Q.dequant_128x128(*wp2[0]), W13)
    a = OL.forward(x, ids, w, 0, L, wmx, mx=True)
    b = OL.forward(x, ids, w, 0, L, wp2, pow2=True)
    for key in ("GU", "h", "Y", "y"):
        assert np.allclose(a[key], b[key], rtol=1e-12, atol=1e-12 * np.max(np.abs(b[key]))), key


def test_forward_chain_close_to_exact():
    """With Gaussian weights the 4-bit grid alone costs about 12% per matrix;
    the chain's output error must be of that order (two weight matrices plus
    FP8 activations), and no larger."""
    rng = np.random.default_rng(7)
    T, d, f, E, L, k = 64, 256, 128, 8, 8, 2
    W13 = bf16(rng.standard_normal((L, 2 * f, d)) * 0.05)
    W2 = bf16(rng.standard_normal((L, d, f)) * 0.05)
    x = bf16(rng.standard_normal((T, d)))
    ids, w = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    wmx = OL.quantize_weights(W13, W2, mx=True)
    ew = max(np.linalg.norm(MX.dequant_mx(*q[:2]) - W) / np.linalg.norm(W) for q, W in zip(wmx, (W13, W2)))
    ex = OL.forward(x, ids, w, 0, L, (W13, W2), exact=True)
    mx = OL.forward(x, ids, w, 0, L, wmx, mx=True)
    rel = np.linalg.norm(mx["y"] - ex["y"]) / np.linalg.norm(ex["y"])
    assert 0.05 < ew < 0.2 and ew < rel < 2.5 * ew, (ew, rel)


def test_training_chain_matches_fp8_on_shared_grid():
    """Weights on the E2M1 grid times one power of two per 128x128 tile, with a
    6 in every 32-block along rows and along columns (the diagonals i = j mod
    32): MX blocks in both directions and the power-of-two 128x128 FP8 tiles
    all hold them exactly, so forward and backward of the MXFP4 chain (its
    dgrad products reading the transposed quantisation) equal the power-of-two
    FP8 chain's."""
    rng = np.random.default_rng(8)
    T, d, f, E, L, k = 64, 256, 128, 8, 8, 2

    def grid_weights(rows, cols):
        w = MX.E2M1_MAG[rng.integers(0, 8, (L, rows, cols))] * np.where(rng.random((L, rows, cols)) < 0.5, -1.0, 1.0)
        i, j = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
        w[:, (i % 32) == (j % 32)] = 6.0
        kexp = rng.integers(-9, -5, (L, rows // 128, cols // 128))
        return w * np.exp2(np.repeat(np.repeat(kexp, 128, axis=1), 128, axis=2))

    W13, W2 = grid_weights(2 * f, d), grid_weights(d, f)
    x = bf16(rng.standard_normal((T, d)))
    dy = bf16(rng.standard_normal((T, d)))
    ids, w = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    wmx = OL.quantize_weights(W13, W2, mx=True)
    wp2 = OL.quantize_weights(W13, W2, pow2=True)
    assert np.array_equal(MX.dequant_mx(*wmx[0][2:]), np.swapaxes(W13, 1, 2))
    fa = OL.forward(x, ids, w, 0, L, wmx, mx=True)
    fb = OL.forward(x, ids, w, 0, L, wp2, pow2=True)
    ba = OL.backward(fa, dy, ids, w, E, wmx, mx=True)
    bb = OL.backward(fb, dy, ids, w, E, wp2, pow2=True)
    for key in ("dx", "dW13", "dW2", "d_logits"):
        assert np.allclose(ba[key], bb[key], rtol=1e-12, atol=1e-12 * np.max(np.abs(bb[key]))), key
