"""Pins for the power-of-two (UE8M0) scale variant of oracle.blockfp8: the
exponent against a brute-force search, the (224, 448] range of amax / s, codes
against an independent division, agreement with the fp32-scale quantiser when
amax / 448 is itself a power of two, padding rows of the 128x1 form, and the
whole forward chain against the unquantised one."""

import numpy as np
import pytest

from oracle import blockfp8 as Q
from oracle import layer as OL
from oracle.numerics import bf16, e4m3_decode, e4m3_encode, f32
from oracle.routing import topk


def _brute_exponent(a):
    """Smallest e in [-200, 200] with a <= 448 * 2^e, by trying them in order."""
    for e in range(-200, 201):
        if a <= 448.0 * 2.0 ** e:
            return e
    raise AssertionError(a)


def test_exponent_brute_force():
    rng = np.random.default_rng(0)
    a = np.exp2(rng.uniform(-60, 120, 500))
    edges = [448.0 * 2.0 ** k * f for k in range(-45, 100, 7)
             for f in (1.0, np.nextafter(1.0, 2.0), np.nextafter(1.0, 0.0), 0.5, 0.75)]
    a = np.concatenate([a, edges, [2.0 ** -40, 224.0, 448.0, 449.0]])
    got = Q.pow2_exponent(a)
    for v, e in zip(a, got):
        assert e == _brute_exponent(float(v)), v


def _check_tiles(x, q, s, tile_of):
    """Every tile: s a power of two, amax / s in (224, 448], codes = e4m3(v / s)."""
    for idx, v in tile_of(x):
        sc = s[idx]
        m, _ = np.frexp(sc)
        assert m == 0.5                                   # a power of two
        a = max(np.max(np.abs(v)), 2.0 ** -40)
        assert 224.0 < a / sc <= 448.0
        ref = e4m3_encode(v / sc)                         # exact division by a power of two
        yield idx, ref


def test_1x128_pow2():
    rng = np.random.default_rng(1)
    x = bf16(rng.standard_normal((5, 384)) * np.exp2(rng.integers(-30, 30, (5, 1))))
    x[2, :128] = 0.0                                      # a zero tile
    q, s = Q.quant_1x128(x, pow2=True)
    tiles = lambda x: (((r, c), x[r, 128 * c:128 * c + 128]) for r in range(5) for c in range(3))
    for (r, c), ref in _check_tiles(x, q, s, tiles):
        assert np.array_equal(q[r, 128 * c:128 * c + 128], ref)
    assert s[2, 0] == 2.0 ** -48 and np.all(q[2, :128] == 0)


def test_128x128_pow2_and_padded_128x1():
    rng = np.random.default_rng(2)
    w = bf16(rng.standard_normal((2, 256, 128)) * 0.02)
    q, s = Q.quant_128x128(w, pow2=True)
    tiles = lambda w: (((e, b, 0), w[e, 128 * b:128 * b + 128, :]) for e in range(2) for b in range(2))
    for (e, b, _), ref in _check_tiles(w, q, s, tiles):
        assert np.array_equal(q[e, 128 * b:128 * b + 128, :], ref)
    src = f32(rng.standard_normal((256, 128)))
    real = np.ones(256, bool)
    real[100:128] = False
    qt, st = Q.quant_128x1_t(src, real, pow2=True)
    z = np.where(real[:, None], src, 0.0)
    tiles_t = lambda z: (((c, b), z[128 * b:128 * b + 128, c]) for c in range(128) for b in range(2))
    for (c, b), ref in _check_tiles(z, qt, st, tiles_t):
        assert np.array_equal(qt[c, 128 * b:128 * b + 128], ref)


def test_pow2_equals_fp32_scales_when_amax_is_448_times_power_of_two():
    rng = np.random.default_rng(3)
    x = f32(rng.uniform(-1, 1, (4, 128)))
    for r in range(4):
        j = rng.integers(0, 128)
        x[r, j] = 448.0 * 2.0 ** int(rng.integers(-10, 10)) * (1 if r % 2 else -1)
        x[r] = np.clip(x[r], -abs(x[r, j]), abs(x[r, j]))
    q1, s1 = Q.quant_1x128(x)
    q2, s2 = Q.quant_1x128(x, pow2=True)
    assert np.array_equal(s1, s2) and np.array_equal(q1, q2)


def test_pow2_dequant_error_bound():
    rng = np.random.default_rng(4)
    x = f32(rng.standard_normal((8, 128)) * np.exp2(rng.integers(-8, 8, (8, 1))))
    q, s = Q.quant_1x128(x, pow2=True)
    dq = e4m3_decode(q) * np.repeat(s, 128, axis=1)
    big = np.abs(x) >= np.repeat(s, 128, axis=1) * 2.0 ** -6   # normal e4m3 range
    assert np.all(np.abs(dq - x)[big] <= np.abs(x)[big] * 2.0 ** -4)


@pytest.mark.parametrize("T,E,k,L", [(96, 8, 2, 8), (200, 16, 4, 6)])
def test_pow2_forward_chain_close_to_exact(T, E, k, L):
    rng = np.random.default_rng(T + L)
    d, f = 256, 256
    x = bf16(rng.standard_normal((T, d)))
    W13 = bf16(rng.standard_normal((L, 2 * f, d)) * 0.05)
    W2 = bf16(rng.standard_normal((L, d, f)) * 0.05)
    ids, w = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    ex = OL.forward(x, ids, w, 0, L, (W13, W2), exact=True)
    fw = OL.forward(x, ids, w, 0, L, OL.quantize_weights(W13, W2, pow2=True), pow2=True)
    rel = np.linalg.norm(fw["y"] - ex["y"]) / np.linalg.norm(ex["y"])
    assert 1e-4 < rel < 0.1                               # quantised, and still the same function
