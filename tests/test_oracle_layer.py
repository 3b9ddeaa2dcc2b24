"""Pins for oracle.layer: the forward and backward chain (with quantisation and
rounding switched off) against torch fp64 autograd of the textbook MoE layer, and
the FP8 chain against the exact one (context-level agreement)."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as LY
from oracle.numerics import bf16
from oracle.routing import topk


def _torch_layer(x, logits, W13, W2, ids, e0, L, dy):
    """Textbook MoE layer written with torch ops, differentiated by autograd."""
    x = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    lg = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    W13 = torch.tensor(W13, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(W2, dtype=torch.float64, requires_grad=True)
    ids_t = torch.from_numpy(ids.astype(np.int64))
    w = torch.softmax(torch.gather(lg, 1, ids_t), dim=1)
    f = W13.shape[1] // 2
    T, k = ids.shape
    y = torch.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j]) - e0
            if 0 <= e < L:
                gu = W13[e] @ x[t]
                h = F.silu(gu[:f]) * gu[f:]
                y = y.index_add(0, torch.tensor([t]), (w[t, j] * (W2[e] @ h))[None])
    (y * torch.from_numpy(dy)).sum().backward()
    return y.detach().numpy(), x.grad.numpy(), lg.grad.numpy(), W13.grad.numpy(), W2.grad.numpy(), w.detach().numpy()


@pytest.mark.parametrize("T,E,k,e0,L", [(40, 4, 2, 0, 4), (48, 8, 3, 2, 4)])
def test_exact_chain_vs_autograd(T, E, k, e0, L):
    rng = np.random.default_rng(T + E)
    d, f = 128, 128
    x = rng.standard_normal((T, d))
    lg = rng.standard_normal((T, E))
    W13 = rng.standard_normal((L, 2 * f, d)) * 0.1
    W2 = rng.standard_normal((L, d, f)) * 0.1
    dy = rng.standard_normal((T, d))
    ids, _ = topk(lg.astype(np.float32), k)
    y_r, dx_r, dl_r, dW13_r, dW2_r, w_t = _torch_layer(x, lg, W13, W2, ids, e0, L, dy)
    fw = LY.forward(x, ids, w_t, e0, L, (W13, W2), exact=True)
    bw = LY.backward(fw, dy, ids, w_t, E, (W13, W2), exact=True)
    assert np.allclose(fw["y"], y_r, rtol=1e-10, atol=1e-12)
    assert np.allclose(bw["dx"], dx_r, rtol=1e-10, atol=1e-12)
    assert np.allclose(bw["dW13"], dW13_r, rtol=1e-10, atol=1e-12)
    assert np.allclose(bw["dW2"], dW2_r, rtol=1e-10, atol=1e-12)
    if e0 == 0 and L == E:       # router gradient is complete only with every expert local
        assert np.allclose(bw["d_logits"], dl_r, rtol=1e-10, atol=1e-12)


def test_fp8_chain_close_to_exact():
    rng = np.random.default_rng(11)
    T, E, k, d, f = 128, 8, 2, 128, 256
    x = bf16(rng.standard_normal((T, d)))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    W13 = bf16(rng.standard_normal((E, 2 * f, d)) * 0.02)
    W2 = bf16(rng.standard_normal((E, d, f)) * 0.02)
    dy = bf16(rng.standard_normal((T, d)))
    ids, w = topk(lg, k)
    wq = LY.quantize_weights(W13, W2)
    fq = LY.forward(x, ids, w, 0, E, wq)
    fe = LY.forward(x, ids, w, 0, E, (W13, W2), exact=True)
    rel = np.linalg.norm(fq["y"] - fe["y"]) / np.linalg.norm(fe["y"])
    assert 1e-3 < rel < 0.1          # FP8 costs a few percent, no more
    bq = LY.backward(fq, dy, ids, w, E, wq)
    be = LY.backward(fe, dy, ids, w, E, (W13, W2), exact=True)
    for key in ("dx", "dW13", "dW2", "d_logits"):
        rel = np.linalg.norm(bq[key] - be[key]) / np.linalg.norm(be[key])
        assert rel < 0.15, key
