"""The MoE expert layer on one GPU's share of experts: forward and training backward.

Forward (expert e, real row r holding token t, slot j):
    X_r  = x[t]                           (bf16 values)
    GU_r = X_r @ W13[e]^T                 W13 = [W_gate; W_up], shape [2f, d]
    h_r  = silu(G_r) * U_r                (SwiGLU, no bias)
    Y_r  = h_r @ W2[e]^T                  W2 shape [d, f]
    y[t] = sum_j w[t, j] * Y_r            (combine)
with block-scaled FP8 operands for both GEMMs ("RL at 1T scale", section "FP8
Training": DeepSeek-V3 style block scaling): X and h quantised 1x128 along K,
weights 128x128.

Backward, given dy [T, d]:
    dY_r        = w[t, j] * dy[t]                   d_gate[t, j] = <dy[t], Y_r>
    dH_r        = dY_r @ W2[e]
    dG          = dH * U * s(G) * (1 + G (1 - s(G))),  dU = dH * silu(G)   (s = sigmoid)
    dX_r        = [dG, dU]_r @ W13[e]               dx[t] = sum_j dX_r
    dW2[e]      = sum_r dY_r^T h_r                  dW13[e] = sum_r [dG, dU]_r^T X_r
    d_logits    = softmax-over-selection backward of d_gate
In the FP8 form every GEMM operand is re-quantised along that GEMM's contraction
axis: 1x128 along features for the dgrad products, 128x1 along tokens for the
wgrad products.

Rounding points (one reading of the pages, which fix no precision): every GEMM
result is first an fp32 accumulator, so G, U, h and dH are fp32, and h is
quantised from fp32; Y is bf16; y = bf16 of the sum; dY_r is one fp32 multiply;
G and U are saved in bf16 and the backward works from those; dGU and the
recomputed h are fp32 before quantisation; dX, dx, dW13, dW2 are bf16;
d_gate and d_logits are fp32.

``exact=True`` runs the same chain with every quantiser and rounding replaced by
the identity and every GEMM by a plain fp64 product; the tests compare that mode
against torch fp64 autograd to pin the chain's formulas.
"""

import numpy as np

from . import blockfp8, dispatch, gemm, mxfp4
from .numerics import bf16, f32
from .routing import gate_backward


def silu(g):
    return g / (1.0 + np.exp(-g))


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


class _FP8:
    """Block-scaled FP8 operands and the rounding points of the library."""
    r32 = staticmethod(f32)
    r16 = staticmethod(bf16)

    @staticmethod
    def weights(W13, W2):
        return blockfp8.quant_128x128(W13), blockfp8.quant_128x128(W2)

    act = staticmethod(blockfp8.quant_1x128)
    act_t = staticmethod(blockfp8.quant_128x1_t)

    @staticmethod
    def fwd(a, wq, counts, offsets):
        return gemm.grouped_forward(a[0], a[1], counts, offsets, wq[0], wq[1])

    @staticmethod
    def dgrad(a, wq, counts, offsets):
        return gemm.grouped_dgrad(a[0], a[1], counts, offsets, wq[0], wq[1])

    @staticmethod
    def wgrad(at, bt, counts, offsets):
        return gemm.grouped_wgrad(at[0], at[1], bt[0], bt[1], counts, offsets)


class _FP8Pow2(_FP8):
    """The same chain with power-of-two (UE8M0) tile scales everywhere."""

    @staticmethod
    def weights(W13, W2):
        return blockfp8.quant_128x128(W13, pow2=True), blockfp8.quant_128x128(W2, pow2=True)

    act = staticmethod(lambda v: blockfp8.quant_1x128(v, pow2=True))
    act_t = staticmethod(lambda v, real: blockfp8.quant_128x1_t(v, real, pow2=True))


class _MXFP4(_FP8Pow2):
    """MXFP4 expert weights (E2M1 codes, one E8M0 scale per 32 values along the
    contraction axis) with power-of-two FP8 activations and gradients.  Each
    weight matrix is quantised twice, as MX blocks run along the contraction
    axis of the product that reads them: W [N, K] along K for the forward, and
    its transpose [K, N] along N for the dgrad product.  The weight-gradient
    products read no weights and stay FP8 (128x1 power-of-two operands)."""

    @staticmethod
    def weights(W13, W2):
        def both(W):
            return mxfp4.quant_mx(W) + mxfp4.quant_mx(np.swapaxes(np.asarray(W, np.float64), -1, -2))
        return both(W13), both(W2)

    @staticmethod
    def fwd(a, wq, counts, offsets):
        return mxfp4.grouped_forward(a[0], a[1], counts, offsets, wq[0], wq[1])

    @staticmethod
    def dgrad(a, wq, counts, offsets):
        # the transposed weights [K, N] play the forward weights' part
        return mxfp4.grouped_forward(a[0], a[1], counts, offsets, wq[2], wq[3])


class _Exact:
    """Unquantised fp64 chain (for the autograd pin)."""
    r32 = staticmethod(lambda v: np.asarray(v, dtype=np.float64))
    r16 = r32

    @staticmethod
    def weights(W13, W2):
        return np.asarray(W13, np.float64), np.asarray(W2, np.float64)

    act = staticmethod(lambda v: np.asarray(v, np.float64))

    @staticmethod
    def act_t(v, real):
        return np.where(np.asarray(real)[:, None], v, 0.0).T

    @staticmethod
    def _segments(counts, offsets):
        for e in range(len(counts)):
            n = int(counts[e])
            if n:
                yield e, slice(int(offsets[e]), int(offsets[e]) + n)

    @classmethod
    def fwd(cls, a, w, counts, offsets):
        out = np.zeros((a.shape[0], w.shape[1]))
        for e, r in cls._segments(counts, offsets):
            out[r] = a[r] @ w[e].T
        return out

    @classmethod
    def dgrad(cls, a, w, counts, offsets):
        out = np.zeros((a.shape[0], w.shape[2]))
        for e, r in cls._segments(counts, offsets):
            out[r] = a[r] @ w[e]
        return out

    @staticmethod
    def wgrad(at, bt, counts, offsets):
        L = len(counts)
        out = np.zeros((L, at.shape[0], bt.shape[0]))
        for e in range(L):
            c = slice(int(offsets[e]), int(offsets[e + 1]))
            out[e] = at[:, c] @ bt[:, c].T
        return out


def _chain(exact, pow2, mx=False):
    if mx:
        return _MXFP4
    return _Exact if exact else (_FP8Pow2 if pow2 else _FP8)


def quantize_weights(W13, W2, pow2=False, mx=False):
    """128x128 FP8 weights: ((W13q, W13s), (W2q, W2s)); pow2 for power-of-two
    scales.  mx: MXFP4 weights, per matrix (codes, E8M0 scale codes, codes of
    the transpose, its scale codes), codes unpacked."""
    return _chain(False, pow2, mx).weights(W13, W2)


def forward(x, ids, w, e0, L, wq, exact=False, pow2=False, mx=False):
    """x [T, d] bf16 values, ids [T, k], gates w [T, k]; wq from quantize_weights
    (or the fp64 weights when exact).  pow2: every activation tile scale is a
    power of two (the weights must be quantised the same way).  mx: MXFP4
    weights with power-of-two FP8 activations.  Returns a dict of every
    intermediate."""
    B = _chain(exact, pow2, mx)
    x = np.asarray(x, dtype=np.float64)
    T, k = np.asarray(ids).shape
    counts, offsets, row_pair, pair_row = dispatch.permute_index(ids, e0, L)
    Xp = dispatch.gather_rows(x, row_pair, k)
    Xa = B.act(Xp)
    GU = B.fwd(Xa, wq[0], counts, offsets)
    f = GU.shape[1] // 2
    G, U = B.r32(GU[:, :f]), B.r32(GU[:, f:])
    h = B.r32(silu(G) * U)
    ha = B.act(h)
    Y = B.r16(B.fwd(ha, wq[1], counts, offsets))
    y = dispatch.combine(Y, pair_row, w) if not exact else _combine_exact(Y, pair_row, w)
    return dict(counts=counts, offsets=offsets, row_pair=row_pair, pair_row=pair_row,
                Xp=Xp, Xa=Xa, GU=GU, G=G, U=U, h=h, ha=ha, Y=Y, y=y, k=k)


def _combine_exact(Y, pair_row, w):
    T, k = pair_row.shape
    y = np.zeros((T, Y.shape[1]))
    for j in range(k):
        r = pair_row[:, j]
        m = r >= 0
        y[m] += (1.0 if w is None else np.asarray(w, np.float64)[m, j][:, None]) * Y[r[m]]
    return y


def backward(fw, dy, ids, w, E, wq, exact=False, pow2=False, mx=False):
    """Training backward of ``forward``'s result ``fw`` for upstream gradient dy [T, d]
    (mx: MXFP4 weights from quantize_weights(..., mx=True))."""
    B = _chain(exact, pow2, mx)
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = fw["k"]
    row_pair, pair_row = fw["row_pair"], fw["pair_row"]
    counts, offsets = fw["counts"], fw["offsets"]
    real = row_pair >= 0
    t_r = row_pair[real] // k
    j_r = row_pair[real] % k
    n_rows, d = fw["Xp"].shape

    # combine backward
    dYp = np.zeros((n_rows, d))
    dYp[real] = B.r32(w[t_r, j_r][:, None] * dy[t_r])
    d_gate = np.zeros(w.shape)
    d_gate[t_r, j_r] = B.r32(np.sum(dy[t_r] * fw["Y"][real], axis=1))

    # dgrad through W2, then dSwiGLU from the saved (bf16) G, U
    dH = B.r32(B.dgrad(B.act(dYp), wq[1], counts, offsets))
    Gs, Us = B.r16(fw["G"]), B.r16(fw["U"])
    sg = sigmoid(Gs)
    dG = dH * Us * sg * (1.0 + Gs * (1.0 - sg))
    dU = dH * Gs * sg
    dGU = np.zeros((n_rows, dG.shape[1] * 2))
    dGU[real] = B.r32(np.concatenate([dG, dU], axis=1)[real])
    Hr = B.r32(Gs * sg * Us)

    # dgrad through W13, unpermute-sum
    dX = B.r16(B.dgrad(B.act(dGU), wq[0], counts, offsets))
    dx = dispatch.combine(dX, pair_row, None) if not exact else _combine_exact(dX, pair_row, None)

    # wgrad, operands quantised along tokens
    dW2 = B.r16(B.wgrad(B.act_t(dYp, real), B.act_t(Hr, real), counts, offsets))
    dW13 = B.r16(B.wgrad(B.act_t(dGU, real), B.act_t(fw["Xp"], real), counts, offsets))

    d_logits = gate_backward(d_gate, w, ids, E) if not exact else _gate_bwd_exact(d_gate, w, ids, E)
    return dict(dYp=dYp, d_gate=d_gate, dH=dH, dGU=dGU, Hr=Hr, dX=dX, dx=dx,
                dW2=dW2, dW13=dW13, d_logits=d_logits)


def _gate_bwd_exact(g, w, ids, E):
    T, k = g.shape
    dsel = w * (g - np.sum(w * g, axis=1, keepdims=True))
    out = np.zeros((T, E))
    np.add.at(out, (np.repeat(np.arange(T), k), np.asarray(ids, np.int64).ravel()), dsel.ravel())
    return out
