"""Routing: top-k selection with softmax gates, and Router Replay (R3).

Top-k (plain definition).  For token t, experts are ordered by the key
(-logit[t, e], e) with IEEE comparison, so -0.0 == +0.0 and equal logits fall back
to the lower expert id.  ids[t, 0..k-1] are the first k experts in that order
(slot 0 holds the largest logit).  Gates are the softmax restricted to the k
selected logits, which equals the full softmax renormalised over the selection:
    m = max_j l_j,   w_j = exp(l_j - m) / sum_j' exp(l_j' - m)
evaluated in fp64 and stored as fp32.

Router Replay ("RL at 1T scale", section "Router Replay"): routing decisions
captured during inference are replayed in the trainer instead of recomputing
top-k.  The record is shaped [num_layers, top_k, seq_len]; a chunk of T tokens
starting at sequence position s0 of layer l replays
    ids[t, j] = R[l, j, s0 + t]
verbatim, keeping the recorded slot order.  Gates are recomputed as the softmax of
the trainer's logits gathered at the replayed ids; the max shift is the max over
the k gathered logits, because under replay slot 0 need not hold the largest.
A token whose ids leave [0, E) is flagged BAD_ID and gets all-zero gates; a token
with a repeated id is flagged DUP_ID and keeps its computed gates.
"""

import numpy as np

from .numerics import f32

FLAG_BAD_ID = 1
FLAG_DUP_ID = 2


def softmax_gates(sel_logits):
    """fp32 gates from the k selected (fp32) logits of each token, in fp64."""
    v = np.asarray(sel_logits, dtype=np.float64)
    m = np.max(v, axis=1, keepdims=True)
    ex = np.exp(v - m)
    return f32(ex / np.sum(ex, axis=1, keepdims=True))


def topk(logits, k):
    """logits fp32 [T, E] -> ids int32 [T, k], gates fp32-valued float64 [T, k]."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    eid = np.arange(E)
    for t in range(T):
        # np.lexsort sorts by the last key first; float compare treats -0 == +0
        order = np.lexsort((eid, -logits[t]))
        ids[t] = order[:k]
    w = softmax_gates(np.take_along_axis(logits, ids.astype(np.int64), axis=1))
    return ids, w


def capture(ids_per_layer):
    """Inference-side capture: stack each layer's ids [T, k] into [NL, k, T]."""
    return np.ascontiguousarray(np.stack([np.asarray(i).T for i in ids_per_layer]).astype(np.int32))


def replay(rec, layer, s0, T, logits):
    """rec int32 [NL, k, S]; logits fp32 [T, E] for tokens s0 .. s0+T-1 of the layer.

    Returns ids int32 [T, k], gates [T, k], status flag bits (int)."""
    rec = np.asarray(rec)
    logits = np.asarray(logits, dtype=np.float64)
    E = logits.shape[1]
    ids = np.ascontiguousarray(rec[layer, :, s0:s0 + T].T).astype(np.int32)
    k = ids.shape[1]
    bad = np.any((ids < 0) | (ids >= E), axis=1)
    srt = np.sort(ids, axis=1)
    dup = np.any(srt[:, 1:] == srt[:, :-1], axis=1) if k > 1 else np.zeros(len(ids), bool)
    w = np.zeros((len(ids), k), dtype=np.float64)
    good = ~bad
    if np.any(good):
        g = np.take_along_axis(logits[good], ids[good].astype(np.int64), axis=1)
        w[good] = softmax_gates(g)
    status = (FLAG_BAD_ID if np.any(bad) else 0) | (FLAG_DUP_ID if np.any(dup) else 0)
    return ids, w, status


def gate_backward(d_gate, w, ids, E):
    """Backward of the softmax over the selected logits.

    d_logits[t, ids[t, j]] = w_j * (g_j - sum_j' w_j' g_j'), zero at unselected
    experts (the selection itself is piecewise constant); a repeated id sums its
    slots.  fp64, stored fp32."""
    g = np.asarray(d_gate, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, k = g.shape
    dsel = w * (g - np.sum(w * g, axis=1, keepdims=True))
    out = np.zeros((T, E), dtype=np.float64)
    rows = np.repeat(np.arange(T), k)
    np.add.at(out, (rows, np.asarray(ids, dtype=np.int64).ravel()), dsel.ravel())
    return f32(out)
