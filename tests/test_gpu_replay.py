"""Router Replay at its full size, through the C ABI: the recorded expert ids
[num_layers=4, top_k=8, seq_len=131072] ("RL at 1T scale", section "Router
Replay": routing decisions captured at inference are replayed in the trainer,
the record staying a device tensor).

* Two 16384-token chunks, (layer 0, chunk 0) and (layer 3, chunk 7), replayed
  through the forward exactly as the benchmark's replay leg launches it: ids,
  gates and every permutation index against the oracle (ids and indices
  bit-exact), then GEMM1 at full K, GEMM2 and the combine on sampled rows of the
  hottest, a middle and the coldest local expert.
* The capture side: top-k over every chunk of all four layers writes the record
  in place; replaying every chunk from it gives back the routed ids and gates
  bit for bit, and two chunks of the record equal the oracle's top-k."""

import numpy as np
import pytest
import torch

from oracle import dispatch as OD
from oracle import routing as OR
from moe_expert_layer_r3_amd import ops, synth
from gpu_util import DEV, gpu, np64, npi, say
import layer_checks as LC

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def record():
    wl = synth.WORKLOADS["replay"]
    say("replay: generating the [4, 8, 131072] record")
    rec = synth.replay_record(wl)
    return wl, rec


@pytest.mark.parametrize("layer,chunk", [(0, 0), (3, 7)])
def test_replay_chunk_full_size(record, layer, chunk):
    from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights
    wl, rec = record
    s0 = chunk * wl.T
    say(f"replay layer {layer} chunk {chunk}: inputs")
    lg = synth.logits(wl, layer=layer, t0=s0)
    x = synth.x(wl, layer=layer, t0=s0)
    W13 = synth.weights(wl, "w13", layer=layer)
    W2 = synth.weights(wl, "w2", layer=layer)
    wts = quantize_weights(W13.to(DEV), W2.to(DEV))
    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=DEV)
    rec_d = gpu(rec)
    say(f"replay layer {layer} chunk {chunk}: GPU forward")
    plan.forward(x.to(DEV), gpu(lg), wts, replay=(rec_d, layer, s0))
    torch.cuda.synchronize()
    del rec_d
    rids, rw, rst = OR.replay(rec, layer, s0, wl.T, lg)
    assert rst == 0 and int(plan.status.item()) == 0
    assert np.array_equal(npi(plan.ids), rids)
    assert np.max(np.abs(np64(plan.w) - rw)) <= 1e-6
    c, o, rp, pr = OD.permute_index(rids, wl.e0, wl.L)
    assert np.array_equal(npi(plan.counts), c) and np.array_equal(npi(plan.offsets), o)
    assert np.array_equal(npi(plan.pair_row), pr)
    n = int(o[-1])
    assert np.array_equal(npi(plan.row_pair)[:n], rp)
    say(f"replay layer {layer} chunk {chunk}: {int(c.sum())} local pairs (counts {c.max()}..{c.min()}), "
        "indices bit-exact")
    experts = (int(np.argmax(c)), int(np.argsort(c)[len(c) // 2]), int(np.argmin(c)))
    h32 = LC.gemm1_h32(plan.xq, plan.xq_s, wts["w13q"], wts["w13s"], plan.counts, plan.offsets,
                       thin_ws=plan.thin_ws)
    LC.check_layer_forward(wl, x, W13, W2, plan, h32, experts, wts=wts, n_rows=16, tok_stride=211,
                           tag=f"replay l{layer} c{chunk}")


def test_capture_replay_roundtrip_full_record():
    """Capture: every chunk of every layer routed by top-k with the record
    written in place; replay: every chunk read back from that record."""
    wl = synth.WORKLOADS["replay"]
    nchunk = wl.seq_len // wl.T
    rec = torch.full((wl.n_layers, wl.k, wl.seq_len), -1, dtype=torch.int32, device=DEV)
    routed = {}
    lgs = {}
    for l in range(wl.n_layers):
        say(f"capture: layer {l}, {nchunk} chunks")
        for c in range(nchunk):
            lg = gpu(synth.logits(wl, layer=l, t0=c * wl.T))
            ids, w = ops.route_topk(lg, wl.k, capture=(rec, l, c * wl.T))
            routed[(l, c)] = (ids, w)
            lgs[(l, c)] = lg
    torch.cuda.synchronize()
    assert int((rec < 0).sum().item()) == 0            # every entry of the record written
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("replay: every chunk")
    for (l, c), (ids0, w0) in routed.items():
        ids, w = ops.replay_load(rec, l, c * wl.T, lgs[(l, c)], status)
        assert torch.equal(ids, ids0), (l, c)
        assert torch.equal(w, w0), (l, c)            # same gate arithmetic in the same order
        assert torch.equal(rec[l, :, c * wl.T:(c + 1) * wl.T].t(), ids0), (l, c)
    assert int(status.item()) == 0
    for l, c in ((0, 0), (3, 7)):
        say(f"capture: oracle top-k of layer {l} chunk {c}")
        rids, rw = OR.topk(npi(lgs[(l, c)]), wl.k)
        assert np.array_equal(npi(rec[l, :, c * wl.T:(c + 1) * wl.T]), rids.T)
        assert np.max(np.abs(np64(routed[(l, c)][1]) - rw)) <= 1e-6
