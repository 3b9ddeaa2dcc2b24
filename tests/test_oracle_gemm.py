"""Pins for oracle.gemm: the fp64 exactness lemma against integer brute force,
single-block and one-hot special cases, and the grouped forms against
dequantise-then-multiply."""

import numpy as np

from oracle import blockfp8 as Q
from oracle import dispatch as D
from oracle import gemm as G
from oracle.numerics import E4M3_VALUES, bf16, f32
from oracle.routing import topk

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
# exact integer value of every code in units of 2^-9
UNITS = {int(c): int(round(E4M3_VALUES[c] * 512)) for c in FINITE}


def _int_brute(qa, qb):
    M, K = qa.shape
    N = qb.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0
            for i in range(K):
                acc += UNITS[int(qa[m, i])] * UNITS[int(qb[n, i])]
            out[m, n] = acc * 2.0 ** -18          # exact: |acc| < 2^53
    return out


def test_exactness_lemma_unit_scales():
    rng = np.random.default_rng(0)
    M, N, K = 3, 4, 384
    qa = rng.choice(FINITE, (M, K))
    qb = rng.choice(FINITE, (N, K))
    ones_a = np.ones((M, K // 128))
    ones_b = np.ones((N, K // 128))
    assert np.array_equal(G.blockscaled_matmul(qa, ones_a, qb, ones_b), _int_brute(qa, qb))
    # extreme codes: every product at the top of the range
    qa = np.full((1, 128), 0x7E, np.uint8)
    qb = np.full((1, 128), 0xFE, np.uint8)
    assert G.blockscaled_matmul(qa, np.ones((1, 1)), qb, np.ones((1, 1)))[0, 0] == -128 * 448.0 * 448.0


def test_single_block_and_one_hot():
    rng = np.random.default_rng(1)
    qa = rng.choice(FINITE, (2, 128))
    qb = rng.choice(FINITE, (5, 128))
    sa = f32(rng.random((2, 1)))
    sb = f32(rng.random((5, 1)))
    got = G.blockscaled_matmul(qa, sa, qb, sb)
    assert np.array_equal(got, (sa * sb.T) * _int_brute(qa, qb))
    onehot = np.zeros((1, 256), np.uint8)
    onehot[0, 130] = 0x38                            # the code of 1.0
    qb2 = rng.choice(FINITE, (6, 256))
    sa2 = np.array([[0.5, 3.0]])
    sb2 = f32(rng.random((6, 2)))
    got = G.blockscaled_matmul(onehot, sa2, qb2, sb2)
    assert np.array_equal(got[0], 3.0 * sb2[:, 1] * E4M3_VALUES[qb2[:, 130]])


def _setup(rng, T=96, E=8, k=2, e0=0, L=8, d=256, f=256):
    ids, _ = topk(rng.standard_normal((T, E)).astype(np.float32), k)
    c, o, rp, pr = D.permute_index(ids, e0, L)
    x = bf16(rng.standard_normal((T, d)))
    Xq, Xs = Q.quant_1x128(D.gather_rows(x, rp, k))
    W = bf16(rng.standard_normal((L, f, d)) * 0.02)
    Wq, Ws = Q.quant_128x128(W)
    return c, o, rp, Xq, Xs, Wq, Ws


def test_grouped_forward_vs_dequant_matmul():
    rng = np.random.default_rng(2)
    c, o, rp, Xq, Xs, Wq, Ws = _setup(rng, e0=2, L=4, E=8)
    got = G.grouped_forward(Xq, Xs, c, o, Wq, Ws)
    A = Q.dequant_1x128(Xq, Xs)
    W = Q.dequant_128x128(Wq, Ws)
    for e in range(4):
        r = slice(o[e], o[e] + c[e])
        ref = A[r] @ W[e].T
        assert np.allclose(got[r], ref, rtol=1e-12, atol=1e-12)
        assert np.all(got[o[e] + c[e]:o[e + 1]] == 0)


def test_grouped_dgrad_vs_dequant_matmul():
    rng = np.random.default_rng(3)
    c, o, rp, Xq, Xs, Wq, Ws = _setup(rng, f=384, d=256)
    # dgrad: A has K = f (the forward out dim)
    A = f32(rng.standard_normal((Xq.shape[0], 384)))
    Aq, As = Q.quant_1x128(A)
    got = G.grouped_dgrad(Aq, As, c, o, Wq, Ws)
    W = Q.dequant_128x128(Wq, Ws)
    Ad = Q.dequant_1x128(Aq, As)
    for e in range(8):
        r = slice(o[e], o[e] + c[e])
        assert np.allclose(got[r], Ad[r] @ W[e], rtol=1e-12, atol=1e-12)


def test_grouped_wgrad_vs_outer_products():
    rng = np.random.default_rng(4)
    c, o, rp, *_ = _setup(rng, T=200, k=3)
    n_rows = len(rp)
    real = rp >= 0
    A = f32(rng.standard_normal((n_rows, 128)))
    B = f32(rng.standard_normal((n_rows, 256)))
    qa, sa = Q.quant_128x1_t(A, real)
    qb, sb = Q.quant_128x1_t(B, real)
    got = G.grouped_wgrad(qa, sa, qb, sb, c, o)
    from oracle.numerics import e4m3_decode
    Ad = e4m3_decode(qa) * np.repeat(sa, 128, axis=1)     # [128, n_rows]
    Bd = e4m3_decode(qb) * np.repeat(sb, 128, axis=1)
    for e in range(8):
        ref = np.zeros((128, 256))
        for r in range(o[e], o[e + 1]):
            ref += np.outer(Ad[:, r], Bd[:, r])
        assert np.allclose(got[e], ref, rtol=1e-12, atol=1e-12)
