"""Pins for oracle.numerics: the e4m3 grid against the OCP spec's table points and
against torch's independent float8_e4m3fn cast; fp32 / bf16 rounding against
numpy's and torch's casts."""

import os

import numpy as np
import pytest
import torch

from oracle import numerics as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_points.txt")


def test_spec_points():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        v = N.E4M3_VALUES[int(code, 16)]
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == float(val) and np.signbit(v) == val.startswith("-")


def test_table_shape():
    v = N.E4M3_VALUES
    assert np.sum(np.isfinite(v)) == 254
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[128:255], -pos)
    assert np.nanmax(v) == 448.0


def test_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(tv) & np.isnan(N.E4M3_VALUES)
    assert np.all(both_nan | (tv == N.E4M3_VALUES))


def test_encode_decode_roundtrip():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(N.e4m3_encode(N.E4M3_VALUES[finite]), finite)


def _torch_e4m3(y32):
    return torch.from_numpy(y32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("exp_lo,exp_hi", [(-12, -2), (-2, 9)])
def test_encode_exhaustive_vs_torch(exp_lo, exp_hi):
    """Every fp32 pattern with exponent in [exp_lo, exp_hi) (both signs of one half
    of the mantissas, all of them for the positive sign).  Covers every rounding
    boundary of the e4m3 grid, subnormals included; |y| <= 448 keeps torch's cast
    out of its NaN-on-overflow branch."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for e in range(exp_lo, exp_hi):
        bits = ((e + 127) << 23) | mant
        y = bits.view(np.float32)
        y = y[np.abs(y) <= 448.0]
        got = N.e4m3_encode(y.astype(np.float64))
        ref = _torch_e4m3(y)
        assert np.array_equal(got, ref), f"exponent {e}"
        yn = -y[::2]
        assert np.array_equal(N.e4m3_encode(yn.astype(np.float64)), _torch_e4m3(yn)), f"exponent {e} negative"


def test_encode_small_and_saturating():
    rng = np.random.default_rng(7)
    tiny = (rng.random(10000) * 2.0 ** -12).astype(np.float32)
    assert np.all(N.e4m3_encode(tiny) == 0)
    assert np.all(N.e4m3_encode(-tiny) == 0x80)
    assert N.e4m3_encode(np.array([-0.0]))[0] == 0x80
    big = np.array([448.0001, 464.0, 465.0, 1e30, 3.4e38])
    assert np.all(N.e4m3_encode(big) == 0x7E)
    assert np.all(N.e4m3_encode(-big) == 0xFE)
    # the midpoint between 2^-10 and 0 ... and ties to even at the bottom of the grid
    assert N.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00       # tie 0 / 2^-9 -> even (0)
    assert N.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02   # tie 1 / 2 -> even (2)
    assert N.e4m3_encode(np.array([432.0]))[0] == 0x7E            # tie 416 / 448 -> 0x7E even


def test_round_binary_fp32_vs_numpy():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))
    # include exact midpoints between fp32 neighbours
    a = rng.standard_normal(20000).astype(np.float32).astype(np.float64)
    mid = a + np.spacing(a.astype(np.float32)).astype(np.float64) / 2
    for v in (x, mid, -mid):
        assert np.array_equal(N.round_binary(v, 24, -126), v.astype(np.float32).astype(np.float64))


def test_bf16_vs_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 1 << 32, 500000, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    ref = torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = N.bf16(y.astype(np.float64))
    ok = (got == ref) | (np.isinf(got) & np.isinf(ref))
    assert np.all(ok)
    # ties: low 16 bits exactly 0x8000
    t = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)
    t = t[np.isfinite(t)]
    reft = torch.from_numpy(t).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    gt = N.bf16(t.astype(np.float64))
    assert np.all((gt == reft) | (np.isinf(gt) & np.isinf(reft)))


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(3)
    v = N.bf16(rng.standard_normal(1000))
    assert np.array_equal(N.bf16_from_bits(N.bf16_bits(v)), v)
