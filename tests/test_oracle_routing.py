"""Pins for oracle.routing: brute-force top-k, tie handling, softmax invariants, the
Router Replay round trip, replay validation, and the gate backward against torch
fp64 autograd."""

import numpy as np
import torch

from oracle import routing as R


def _brute_topk(row, k):
    # Python's sort on (-value, id); -0.0 == 0.0 in Python comparisons too
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def test_topk_brute_force():
    rng = np.random.default_rng(0)
    for T, E, k in [(17, 8, 2), (9, 16, 5), (5, 33, 8), (4, 7, 7), (3, 1, 1)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = R.topk(lg, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk(lg[t], k)


def test_topk_ties_and_signed_zero():
    rng = np.random.default_rng(1)
    lg = rng.integers(0, 3, (64, 16)).astype(np.float32)
    ids, _ = R.topk(lg, 6)
    for t in range(64):
        assert list(ids[t]) == _brute_topk(lg[t], 6)
    z = np.array([[-0.0, 0.0, -0.0, 0.0]], dtype=np.float32)
    ids, w = R.topk(z, 3)
    assert list(ids[0]) == [0, 1, 2]
    assert np.all(w == np.float32(1.0 / 3.0))


def test_topk_nan_and_infinities():
    # NaN after every number, NaNs by id; -inf after every finite value; a NaN
    # in the selection makes the token's gates NaN, -inf gets gate 0
    nan, inf = np.nan, np.inf
    lg = np.array([[nan, 1.0, -inf, nan, -2.0, 0.5],
                   [-inf, -inf, 3.0, nan, -inf, -1.0]], dtype=np.float32)
    ids, w = R.topk(lg, 5)
    assert list(ids[0]) == [1, 5, 4, 2, 0]
    assert list(ids[1]) == [2, 5, 0, 1, 4]
    assert np.all(np.isnan(w[0]))
    # gates are fp32-valued: within one fp32 rounding of the exact value
    assert abs(w[1, 0] - 1.0 / (1.0 + np.exp(-4.0))) < 6e-8 and np.all(w[1, 2:] == 0.0)
    with np.errstate(invalid="ignore"):
        ids, w = R.topk(lg, 6)
    assert list(ids[0]) == [1, 5, 4, 2, 0, 3]


def test_topk_invariants():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((200, 64)).astype(np.float32)
    ids, w = R.topk(lg, 8)
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)
    for t in range(200):
        assert len(set(ids[t])) == 8
        rest = np.setdiff1d(np.arange(64), ids[t])
        assert np.all(lg[t, rest] <= sel[t, -1])
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-6)
    # gates are the softmax over the selection: compare with torch fp64
    ref = torch.softmax(torch.from_numpy(sel.astype(np.float64)), dim=1).numpy()
    assert np.array_equal(w, ref.astype(np.float32).astype(np.float64))
    ids1, w1 = R.topk(lg, 1)
    assert np.all(w1 == 1.0) and np.array_equal(ids1[:, 0], np.argmax(lg, axis=1))


def test_equal_logits_uniform_gates():
    lg = np.full((3, 10), 0.25, dtype=np.float32)
    ids, w = R.topk(lg, 4)
    assert np.all(ids == np.arange(4)) and np.all(w == np.float32(0.25))


def test_replay_roundtrip():
    """Replay of a captured record reproduces the routing bitwise."""
    rng = np.random.default_rng(3)
    NL, T, E, k = 3, 50, 32, 4
    lgs = [rng.standard_normal((T, E)).astype(np.float32) for _ in range(NL)]
    routed = [R.topk(l, k) for l in lgs]
    rec = R.capture([r[0] for r in routed])
    assert rec.shape == (NL, k, T) and rec.dtype == np.int32
    for l in range(NL):
        for s0, n in [(0, T), (7, 20), (T - 1, 1)]:
            ids, w, st = R.replay(rec, l, s0, n, lgs[l][s0:s0 + n])
            assert st == 0
            assert np.array_equal(ids, routed[l][0][s0:s0 + n])
            assert np.array_equal(w, routed[l][1][s0:s0 + n])


def test_replay_slab_and_max_shift():
    rng = np.random.default_rng(4)
    rec = np.stack([np.stack([rng.permutation(16)[:3] for _ in range(40)]).T for _ in range(2)]).astype(np.int32)
    lg = rng.standard_normal((10, 16)).astype(np.float32)
    ids, w, st = R.replay(rec, 1, 5, 10, lg)
    assert st == 0 and np.array_equal(ids, rec[1, :, 5:15].T)
    g = np.take_along_axis(lg, ids.astype(np.int64), axis=1).astype(np.float64)
    ref = torch.softmax(torch.from_numpy(g), dim=1).numpy()
    assert np.array_equal(w, ref.astype(np.float32).astype(np.float64))


def test_replay_flags():
    rec = np.array([[[0, 1, 2, 3], [1, 9, 2, -1]]], dtype=np.int32)   # [1, k=2, S=4]
    lg = np.zeros((4, 8), dtype=np.float32)
    ids, w, st = R.replay(rec, 0, 0, 4, lg)
    assert st == R.FLAG_BAD_ID | R.FLAG_DUP_ID
    assert np.all(w[1] == 0) and np.all(w[3] == 0)       # tokens 1 (id 9) and 3 (id -1)
    assert np.all(w[0] == 0.5) and np.all(w[2] == 0.5)   # token 2 is (2, 2): duplicate, gates kept
    rec2 = np.array([[[0, 1], [0, 2]]], dtype=np.int32)
    _, w2, st2 = R.replay(rec2, 0, 0, 2, lg[:2])
    assert st2 == R.FLAG_DUP_ID and np.all(w2 == 0.5)


def test_gate_backward_vs_autograd():
    rng = np.random.default_rng(5)
    T, E, k = 20, 12, 3
    lg = rng.standard_normal((T, E))
    ids, _ = R.topk(lg.astype(np.float32), k)
    g = rng.standard_normal((T, k))
    lt = torch.tensor(lg, dtype=torch.float64, requires_grad=True)
    sel = torch.gather(lt, 1, torch.from_numpy(ids.astype(np.int64)))
    wt = torch.softmax(sel, dim=1)
    (wt * torch.from_numpy(g)).sum().backward()
    got = R.gate_backward(g, wt.detach().numpy(), ids, E)
    assert np.allclose(got, lt.grad.numpy(), rtol=0, atol=1e-7)
    for t in range(T):
        assert np.all(np.delete(got[t], ids[t]) == 0)
