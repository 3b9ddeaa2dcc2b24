"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    """torch tensor (bf16/fp32/...) -> float64 numpy on the host."""
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def npi(t):
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        return 0.0 if np.all(got == 0) else np.inf
    return float(np.linalg.norm(got - ref) / nr)


def gpu(x, dtype=None):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        x = x.to(dtype)
    return x.contiguous().to(DEV)


def bf16_tensor(vals):
    """float64 numpy values that are bf16-exact -> bf16 torch tensor on the GPU."""
    return gpu(torch.from_numpy(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16))


def ids_for_counts(counts, k, E, e0, rng):
    """ids [T, k] (distinct per token) whose local experts e0..e0+L-1 receive exactly
    `counts` pairs; remaining slots take non-local experts.  T = max needed."""
    L = len(counts)
    T = max(max(counts), 1)
    assert all(c <= T for c in counts) and E - L >= k
    ids = np.empty((T, k), dtype=np.int32)
    nonlocal_pool = np.array([e for e in range(E) if not (e0 <= e < e0 + L)])
    for t in range(T):
        loc = [e0 + e for e in range(L) if t < counts[e]][:k]
        rest = rng.choice(nonlocal_pool, k - len(loc), replace=False)
        row = np.array(loc + list(rest), dtype=np.int32)
        rng.shuffle(row)
        ids[t] = row
    return ids
