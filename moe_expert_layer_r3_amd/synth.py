"""Seeded synthetic inputs for the MoE layer workloads (shared by tests, bench and
smoke; holds none of the layer's arithmetic).

Every tensor comes from its own numpy PCG64 stream
``np.random.default_rng([0, cfg, tensor_id, *sub])`` so that any expert's weights
or any block of rows can be regenerated alone.  Normals are drawn in fp32, scaled
in fp32 and rounded to bf16 (round to nearest even) where bf16 is specified.

Workloads (the pages train GLM-5 on agentic SWE tasks at up to 131k tokens; no
weights, tasks or routing traces of that run exist here, so these seeded shapes
stand in for them):
  tiny      T=128,   d=128,  f=256,  E=8,   L=8  (all local), k=2, forward
  ep8       T=8192,  d=7168, f=2048, E=256, L=32 (experts 0-31), k=8, forward
  hotspot   as ep8, logits N(0,1) + b_e with b_e = -1.2 ln(e+1) (Zipf-like
            popularity, expert 0 hottest), forward
  replay    recorded ids [4, 8, 131072]: per token 8 distinct ids drawn by
            Gumbel-top-8 of -1.1 ln(e+1) + Gumbel noise (Zipf(1.1) first pick, then
            sampling without replacement), slot = draw order; per layer fp32 N(0,1)
            logits and bf16 x; processed in 16384-token chunks, forward
  train     T=16384, d=7168, f=2048, E=256, L=32, k=8, N(0,1) logits, forward and
            backward with a bf16 N(0,1) upstream gradient
Weights are N(0, 0.02) bf16, W13 = [W_gate; W_up] of shape [L, 2f, d], W2 of shape
[L, d, f].
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np
import torch

TID_LOGITS, TID_X, TID_W13, TID_W2, TID_DY, TID_REC = 0, 1, 2, 3, 4, 5
ROW_BLOCK = 1024


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int
    T: int
    d: int
    f: int
    E: int
    L: int
    k: int
    e0: int = 0
    bias: float = 0.0          # logits += -bias * ln(e + 1)
    n_layers: int = 0          # replay only
    seq_len: int = 0           # replay only
    rec_zipf: float = 0.0      # replay only
    backward: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", 1, T=128, d=128, f=256, E=8, L=8, k=2, backward=True),
    "ep8": Workload("ep8", 2, T=8192, d=7168, f=2048, E=256, L=32, k=8),
    "hotspot": Workload("hotspot", 3, T=8192, d=7168, f=2048, E=256, L=32, k=8, bias=1.2),
    "replay": Workload("replay", 4, T=16384, d=7168, f=2048, E=256, L=32, k=8,
                       n_layers=4, seq_len=131072, rec_zipf=1.1),
    "train": Workload("train", 5, T=16384, d=7168, f=2048, E=256, L=32, k=8, backward=True),
}


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def rng(cfg, tid, *sub):
    return np.random.default_rng([0, cfg, tid, *sub])


def _normal_bf16_rows(cfg, tid, sub, rows, cols, std, out, b0=0):
    """Fill torch bf16 ``out`` [rows, cols] from per-ROW_BLOCK streams (row
    block b of ``out`` from stream b0 + b)."""
    def blk(b):
        r0 = b * ROW_BLOCK
        r1 = min(rows, r0 + ROW_BLOCK)
        z = rng(cfg, tid, *sub, b0 + b).standard_normal((ROW_BLOCK, cols), dtype=np.float32)[:r1 - r0]
        if std != 1.0:
            z *= np.float32(std)
        out[r0:r1] = torch.from_numpy(z).to(torch.bfloat16)
    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(blk, range(nb)))
    return out


def logits(w: Workload, layer=0, t0=0, T=None):
    """fp32 [T, E] router logits (rows t0 .. t0+T-1; replay: of the given layer)."""
    T = w.T if T is None else T
    out = np.empty((T, w.E), dtype=np.float32)
    sub = (layer,) if w.n_layers else ()
    b0, b1 = t0 // ROW_BLOCK, (t0 + T + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        z = rng(w.cfg, TID_LOGITS, *sub, b).standard_normal((ROW_BLOCK, w.E), dtype=np.float32)
        lo, hi = max(t0, b * ROW_BLOCK), min(t0 + T, (b + 1) * ROW_BLOCK)
        out[lo - t0:hi - t0] = z[lo - b * ROW_BLOCK:hi - b * ROW_BLOCK]
    if w.bias:
        out += (-w.bias * np.log(np.arange(1, w.E + 1, dtype=np.float64))).astype(np.float32)
    return out


def x(w: Workload, layer=0, t0=0, T=None):
    """bf16 torch tensor [T, d] of activations; t0 must be a multiple of 1024."""
    T = w.T if T is None else T
    assert t0 % ROW_BLOCK == 0
    out = torch.empty((T, w.d), dtype=torch.bfloat16)
    sub = (layer,) if w.n_layers else ()
    def blk(b):
        r0 = b * ROW_BLOCK
        r1 = min(T, r0 + ROW_BLOCK)
        z = rng(w.cfg, TID_X, *sub, (t0 // ROW_BLOCK) + b).standard_normal((ROW_BLOCK, w.d), dtype=np.float32)
        out[r0:r1] = torch.from_numpy(z[:r1 - r0]).to(torch.bfloat16)
    nb = (T + ROW_BLOCK - 1) // ROW_BLOCK
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(blk, range(nb)))
    return out


def dy(w: Workload, t0=0, T=None):
    """bf16 torch tensor [T, d] upstream gradient of tokens t0 .. t0+T-1; t0 must
    be a multiple of 1024."""
    T = w.T if T is None else T
    assert t0 % ROW_BLOCK == 0
    out = torch.empty((T, w.d), dtype=torch.bfloat16)
    return _normal_bf16_rows(w.cfg, TID_DY, (), T, w.d, 1.0, out, b0=t0 // ROW_BLOCK)


def expert_weights(w: Workload, which, e, layer=0):
    """bf16 torch tensor of one expert: which='w13' -> [2f, d], 'w2' -> [d, f]."""
    tid, shape = (TID_W13, (2 * w.f, w.d)) if which == "w13" else (TID_W2, (w.d, w.f))
    sub = (layer, e) if w.n_layers else (e,)
    z = rng(w.cfg, tid, *sub).standard_normal(shape, dtype=np.float32)
    z *= np.float32(0.02)
    return torch.from_numpy(z).to(torch.bfloat16)


def weights(w: Workload, which, layer=0, experts=None):
    """bf16 torch tensor [L, ...] of all local experts' weights (threaded)."""
    experts = list(range(w.L)) if experts is None else list(experts)
    shape = (2 * w.f, w.d) if which == "w13" else (w.d, w.f)
    out = torch.empty((len(experts), *shape), dtype=torch.bfloat16)
    def one(i):
        out[i] = expert_weights(w, which, experts[i], layer)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(experts))))
    return out


def replay_record(w: Workload, seq_len=None):
    """int32 [n_layers, k, seq_len] recorded expert ids (Gumbel-top-k sampling)."""
    S = w.seq_len if seq_len is None else seq_len
    rec = np.empty((w.n_layers, w.k, S), dtype=np.int32)
    base = -w.rec_zipf * np.log(np.arange(1, w.E + 1, dtype=np.float64))

    def blk(lb):
        l, b = lb
        r0, r1 = b * ROW_BLOCK, min(S, (b + 1) * ROW_BLOCK)
        u = rng(w.cfg, TID_REC, l, b).random((r1 - r0, w.E))
        pert = base[None, :] - np.log(-np.log(np.maximum(u, 1e-300)))
        part = np.argpartition(-pert, w.k - 1, axis=1)[:, :w.k]
        o = np.argsort(-np.take_along_axis(pert, part, axis=1), axis=1, kind="stable")
        rec[l, :, r0:r1] = np.take_along_axis(part, o, axis=1).T
    jobs = [(l, b) for l in range(w.n_layers) for b in range((S + ROW_BLOCK - 1) // ROW_BLOCK)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(blk, jobs))
    return rec


def tiny_variant(base: Workload, **kw):
    """A workload with the given fields replaced (reduced shapes for parity tests);
    the seed namespace gets its own cfg id so streams never alias."""
    fields = dict(base.__dict__)
    fields.update(kw)
    fields["cfg"] = kw.get("cfg", 100 + base.cfg)
    return Workload(**fields)
