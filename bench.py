"""Benchmark of the MoE expert layer on one MI355X.

Headline step = one training step of the layer on the EP=8 share of a
256-expert top-8 layer (T=16384 tokens, d=7168, f=2048 SwiGLU, local experts
0-31): the expert weights re-quantised to 128x128 FP8 blocks (they change every
optimizer step), top-k routing, the expert-grouped permutation with fused 1x128
quantisation, grouped GEMM1 with the fused SwiGLU + quantisation epilogue
saving bf16 G/U, grouped GEMM2, the weighted combine, then the backward:
combine backward (dY 1x128 + d_gate), dY and x re-quantised 128x1 along tokens,
dgrad through W2 + SwiGLU backward (dGU 1x128 / 128x1, H 128x1), dgrad through
W13 + unpermute-sum, both wgrad products and the gate backward.  Inputs are
seeded synthetic tensors already resident in HBM; two input sets of 0.49 GB
(x, logits, dy) alternate between steps, so no step finds its inputs in the
256 MB last-level cache.  The step is timed twice: launched eagerly with HIP
events around every stage (per-kernel times and the roofline come from these),
and captured into a HIP graph per input set and replayed (ms_per_step and the
throughput; the same kernels without per-launch host cost).

Further legs, reported as sub-objects of the same JSON line, each with the
roofline of its dominant kernel:
  ep8      forward of the T=8192 share (three rotating input sets)
  hotspot  the same forward with Zipf-skewed routing (unequal expert loads)
  replay   Router Replay of a recorded [4, 8, 131072] id tensor: every layer's
           131072 tokens in 16384-token chunks, each layer with its own weights
  pow2 / mxfp4            the ep8 forward with power-of-two (UE8M0) tile scales /
                          MXFP4 expert weights
  train_pow2 / train_mxfp4  the training step with those variants

The oracle (plain numpy fp64, CPU) is timed first, before any GPU use, on the
host cores: the whole training step (routing, permutation, forward, backward)
for the first --cpu-tokens tokens of the headline workload over all 32 local
experts, the rate reported as measured (no extrapolation); its 128x128 weight
quantisation runs in an untimed setup, one expert per process."""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
METRIC = "MoE-layer tokens/s + FP8 grouped-GEMM TFLOP/s (% of MFMA peak)"
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="ep8,hotspot,replay,pow2,mxfp4,train_pow2,train_mxfp4",
                    help="comma-separated extra legs (ep8, hotspot, replay, pow2, mxfp4, train_pow2, "
                         "train_mxfp4) or 'none'")
    ap.add_argument("--replay-passes", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="tokens of the headline workload the oracle runs in the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, 5 times: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters against a known
    byte count (1 GiB read and 1 GiB written per dispatch)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}), flush=True)


# ---------------------------------------------------------------- algorithmic work

def _wbytes(n, k, mxfp4):
    """Bytes of one [n, k] weight matrix: FP8 codes + 128x128 fp32 scales, or
    E2M1 codes + one E8M0 scale byte per 32 values."""
    return n * k // 2 + n * (k // 32) if mxfp4 else n * k + (n // 128) * (k // 128) * 4


def _q(n):
    """FP8 codes of n elements + fp32 scales per 128 (1x128 or 128x1 tiles)."""
    return n + n // 128 * 4


def forward_work(P, L, d, f, mxfp4=False):
    """Algorithmic FLOPs and HBM bytes of the two forward grouped GEMMs for P
    local pairs (padding rows not counted)."""
    return {"gemm1": (4.0 * P * d * f, L * _wbytes(2 * f, d, mxfp4) + _q(P * d) + _q(P * f)),
            "gemm2": (2.0 * P * d * f, L * _wbytes(d, f, mxfp4) + _q(P * f) + P * d * 2)}


def train_work(P, R, L, d, f, mxfp4=False):
    """Algorithmic FLOPs and HBM bytes of the six grouped GEMMs of a training
    step: P local pairs, R expert-grouped rows (segments padded to 128, the wgrad
    contraction)."""
    w = lambda n, k: L * _wbytes(n, k, mxfp4)
    return {"gemm1": (4.0 * P * d * f, w(2 * f, d) + _q(P * d) + _q(P * f) + P * 2 * f * 2),   # + saved bf16 G/U
            "gemm2": (2.0 * P * d * f, w(d, f) + _q(P * f) + P * d * 2),
            "dgrad2": (2.0 * P * d * f, _q(P * d) + w(f, d) + P * f * 4),                      # dH fp32
            "dgrad1": (4.0 * P * d * f, _q(P * 2 * f) + w(d, 2 * f) + P * d * 2),              # dX bf16
            "wgrad2": (2.0 * P * d * f, _q(R * d) + _q(R * f) + L * d * f * 2),                # dW2 bf16
            "wgrad13": (4.0 * P * d * f, _q(R * 2 * f) + _q(R * d) + L * 2 * f * d * 2)}       # dW13 bf16


def roofline_of(kernel, flops, nbytes, ms, workload):
    """Roofline entry of one kernel: bound by whichever floor (MFMA or HBM) is
    longer; traffic = HBM bytes per launch measured by rocprofv3 counters when a
    profile of this kernel's current code exists."""
    t_mfma = flops / (FP8_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t = ms * 1e-3
    if t_hbm >= t_mfma:
        r = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": t_hbm / t}
    else:
        r = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": t_mfma / t}
    r["traffic"] = measured_traffic(kernel, workload)
    r["kernel"] = kernel
    r["algorithmic_bytes"] = nbytes
    r["flops"] = flops
    r["ms"] = ms
    return r


def measured_traffic(kernel, workload):
    """HBM bytes per launch of a kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (profiles/<kernel>_<workload>_traffic.json), or None when
    there is none or the kernel's code changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(HERE, "moe_expert_layer_r3_amd", "csrc")
    from moe_expert_layer_r3_amd.prof_summary import code_sha256
    if code_sha256([os.path.join(src, f) for f in rec["sources"]]) != rec["code_sha256"]:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def stage_events(names, steps):
    return {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)] for n in names}


def mean_ms(ev):
    return {n: float(np.mean([a.elapsed_time(b) for a, b in pairs])) for n, pairs in ev.items()}


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def timed(fn, steps):
    """Wall time per call of fn over `steps` calls, bracketed by device syncs."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


# ---------------------------------------------------------------- forward legs

def forward_leg(wl, steps, warmup, dev, pow2=False, mxfp4=False, sets=3):
    from moe_expert_layer_r3_amd import synth
    from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights, weight_buffers

    # `sets` input sets (x, logits) of distinct seeded token blocks, rotated
    # across steps: 3 x 125 MB at the ep8 shape, past the last-level cache
    xs = [synth.x(wl, t0=i * wl.T).to(dev) for i in range(sets)]
    lgs = [torch.from_numpy(synth.logits(wl, t0=i * wl.T)).to(dev) for i in range(sets)]
    W13_d, W2_d = synth.weights(wl, "w13").to(dev), synth.weights(wl, "w2").to(dev)

    # weight quantisation (once per weight version), timed on its own
    wts = None if mxfp4 else weight_buffers(wl.L, wl.d, wl.f, dev)
    wts = quantize_weights(W13_d, W2_d, out=wts, pow2=pow2, mxfp4=mxfp4)
    torch.cuda.synchronize()
    qe0, qe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qe0.record()
    for _ in range(3):
        quantize_weights(W13_d, W2_d, out=wts, pow2=pow2, mxfp4=mxfp4)
    qe1.record()
    torch.cuda.synchronize()
    wquant_ms = qe0.elapsed_time(qe1) / 3
    del W13_d, W2_d
    free()

    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=dev, pow2=pow2, mxfp4=mxfp4)
    for i in range(warmup):
        plan.forward(xs[i % sets], lgs[i % sets], wts)
    ev = stage_events(plan.STAGES, steps)
    ms_eager = timed(lambda i: plan.forward(xs[i % sets], lgs[i % sets], wts,
                                            events={n: ev[n][i] for n in plan.STAGES}), steps)
    kern = mean_ms(ev)
    # the same step captured once per input set into a HIP graph and replayed:
    # the kernels are identical, the per-launch host cost goes away
    graphs = [plan.capture(xs[i], lgs[i], wts) for i in range(sets)]
    for i in range(warmup):
        graphs[i % sets].replay()
    ms = timed(lambda i: graphs[i % sets].replay(), steps)
    del graphs
    Ps = []
    for i in range(sets):                      # pair count of every input set
        plan.forward(xs[i], lgs[i], wts)
        Ps.append(int(plan.counts.sum().item()))
    counts = plan.counts.cpu().numpy()
    P = float(np.mean(Ps))
    work = forward_work(P, wl.L, wl.d, wl.f, mxfp4=mxfp4)
    name = wl.name + ("_pow2" if pow2 else "") + ("_mxfp4" if mxfp4 else "")
    gem = {n: {"ms": kern[n], "tflops": fl / (kern[n] * 1e-3) / 1e12, "gbs": by / (kern[n] * 1e-3) / 1e9,
               "flops": fl, "bytes": by} for n, (fl, by) in work.items()}
    g_fl = sum(fl for fl, _ in work.values())
    g_ms = sum(kern[n] for n in work)
    res = {
        "tokens_per_s": wl.T / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "kernel_ms": kern,
        "weight_quant_ms": wquant_ms,
        "local_pairs": Ps,
        "expert_counts": {"max": int(counts.max()), "mean": float(counts.mean()), "min": int(counts.min())},
        "gemms": gem,
        "gemm_tflops": g_fl / (g_ms * 1e-3) / 1e12,
        "gemm_mfma_frac": g_fl / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "input_sets": sets,
        "roofline": roofline_of("gemm1", *work["gemm1"], kern["gemm1"], name),
    }
    del plan, wts, xs, lgs
    free()
    return res


# ---------------------------------------------------------------- training step

def train_leg(steps, warmup, dev, pow2=False, mxfp4=False, sets=2):
    from moe_expert_layer_r3_amd import synth
    from moe_expert_layer_r3_amd.layer import TrainPlan, capture_graph, quantize_weights, weight_buffers

    wl = synth.WORKLOADS["train"]
    # `sets` input sets (x, logits, dy: 0.49 GB each) of distinct seeded token
    # blocks, alternating between steps
    xs = [synth.x(wl, t0=i * wl.T).to(dev) for i in range(sets)]
    lgs = [torch.from_numpy(synth.logits(wl, t0=i * wl.T)).to(dev) for i in range(sets)]
    dys = [synth.dy(wl, t0=i * wl.T).to(dev) for i in range(sets)]
    W13_d = synth.weights(wl, "w13").to(dev)
    W2_d = synth.weights(wl, "w2").to(dev)
    plan = TrainPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=dev, pow2=pow2, mxfp4=mxfp4)
    tw = plan.transpose_weights  # FP8: the dgrad products read the forward weights, no transposed copy
    wts = None if mxfp4 else weight_buffers(wl.L, wl.d, wl.f, dev, transpose=tw)
    wts = quantize_weights(W13_d, W2_d, transpose=tw, out=wts, pow2=pow2, mxfp4=mxfp4)

    def step(i, events=None):
        if events is not None:
            events["weight_quant"][0].record()
        quantize_weights(W13_d, W2_d, transpose=tw, out=wts, pow2=pow2, mxfp4=mxfp4)
        if events is not None:
            events["weight_quant"][1].record()
        plan.forward(xs[i % sets], lgs[i % sets], wts, events=events)
        plan.backward(xs[i % sets], dys[i % sets], wts, events=events)

    for i in range(warmup):
        step(i)
    names = ("weight_quant",) + plan.STAGES + plan.BWD_STAGES
    ev = stage_events(names, steps)
    ms_eager = timed(lambda i: step(i, {n: ev[n][i] for n in names}), steps)
    kern = mean_ms(ev)
    graphs = [capture_graph(lambda i=i: step(i)) for i in range(sets)]
    for i in range(warmup):
        graphs[i % sets].replay()
    ms = timed(lambda i: graphs[i % sets].replay(), steps)
    del graphs
    Ps, Rs = [], []
    for i in range(sets):
        step(i)
        Ps.append(int(plan.counts.sum().item()))
        Rs.append(int(plan.offsets[-1].item()))
    P, R = float(np.mean(Ps)), float(np.mean(Rs))
    work = train_work(P, R, wl.L, wl.d, wl.f, mxfp4=mxfp4)
    name = "train" + ("_pow2" if pow2 else "") + ("_mxfp4" if mxfp4 else "")
    gem = {n: {"ms": kern[n], "tflops": fl / (kern[n] * 1e-3) / 1e12,
               "mfma_frac": fl / (kern[n] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
               "gbs": by / (kern[n] * 1e-3) / 1e9, "flops": fl, "bytes": by} for n, (fl, by) in work.items()}
    g_fl = sum(fl for fl, _ in work.values())
    g_ms = sum(kern[n] for n in work)
    top = max(work, key=lambda n: kern[n])
    res = {
        "workload": f"{name}: T={wl.T}, d={wl.d}, f={wl.f}, {wl.L} of {wl.E} experts local, top-{wl.k}, "
                    "forward + backward, weights re-quantised each step"
                    + (", power-of-two (UE8M0) tile scales" if pow2 else "")
                    + (", MXFP4 weights (forward and dgrad), FP8 power-of-two activations" if mxfp4 else ""),
        "tokens_per_s": wl.T / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "ms_per_step_excl_weight_quant": ms - kern["weight_quant"],
        "local_pairs": Ps,
        "rows": Rs,
        "kernel_ms": kern,
        "gemms": gem,
        "gemm_tflops": g_fl / (g_ms * 1e-3) / 1e12,
        "gemm_mfma_frac": g_fl / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "input_sets": sets,
        "roofline": roofline_of(top, *work[top], kern[top], name),
    }
    del plan, wts, xs, lgs, dys, W13_d, W2_d
    free()
    return res


# ---------------------------------------------------------------- replay leg

def replay_leg(passes, dev):
    from moe_expert_layer_r3_amd import synth
    from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights, weight_buffers

    wl = synth.WORKLOADS["replay"]
    rec = synth.replay_record(wl)
    rec_d = torch.from_numpy(rec).to(dev)
    nchunk = wl.seq_len // wl.T
    # local pairs of every chunk, straight from the record
    loc = (rec >= wl.e0) & (rec < wl.e0 + wl.L)
    P = loc.reshape(wl.n_layers, wl.k, nchunk, wl.T).sum(axis=(1, 3))          # [layer, chunk]
    layers = []
    for l in range(wl.n_layers):
        wts = weight_buffers(wl.L, wl.d, wl.f, dev)
        quantize_weights(synth.weights(wl, "w13", layer=l).to(dev), synth.weights(wl, "w2", layer=l).to(dev),
                         out=wts)
        xs = [synth.x(wl, layer=l, t0=c * wl.T).to(dev) for c in range(nchunk)]
        lgs = [torch.from_numpy(synth.logits(wl, layer=l, t0=c * wl.T)).to(dev) for c in range(nchunk)]
        layers.append((wts, xs, lgs))
        free()
    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=dev)

    def one_pass(ev=None, i=0):
        for l, (wts, xs, lgs) in enumerate(layers):
            for c in range(nchunk):
                events = None if ev is None else {n: ev[n][i * wl.n_layers * nchunk + l * nchunk + c]
                                                  for n in plan.STAGES}
                plan.forward(xs[c], lgs[c], wts, replay=(rec_d, l, c * wl.T), events=events)

    one_pass()
    ev = stage_events(plan.STAGES, passes * wl.n_layers * nchunk)
    ms = timed(lambda i: one_pass(ev, i), passes)
    flags = int(plan.status.item())
    kern = mean_ms(ev)
    work = forward_work(float(P.mean()), wl.L, wl.d, wl.f)
    g_fl = sum(fl for fl, _ in work.values())
    g_ms = sum(kern[n] for n in work)
    res = {
        "workload": f"replay: record [{wl.n_layers}, {wl.k}, {wl.seq_len}] Zipf({wl.rec_zipf}) ids, "
                    f"{wl.T}-token chunks, d={wl.d}, f={wl.f}, {wl.L} of {wl.E} experts local, forward",
        "layer_tokens_per_s": wl.n_layers * wl.seq_len / (ms * 1e-3),
        "ms_per_pass": ms,
        "kernel_ms_per_chunk": kern,
        "local_pairs_per_chunk": {"mean": float(P.mean()), "min": int(P.min()), "max": int(P.max()),
                                  "total": int(P.sum())},
        "gemm_tflops": g_fl / (g_ms * 1e-3) / 1e12,
        "gemm_mfma_frac": g_fl / (g_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "status_flags": flags,
        "roofline": roofline_of("gemm1", *work["gemm1"], kern["gemm1"], "replay"),
    }
    del plan, layers, rec_d
    free()
    return res


# ---------------------------------------------------------------- host baseline

def _oracle_expert_weights(args):
    """One expert's 128x128 FP8 weights quantised by the oracle (process-pool
    worker of the baseline's untimed setup)."""
    from moe_expert_layer_r3_amd import synth
    from oracle import blockfp8 as OQ
    wname, e = args
    wl = synth.WORKLOADS[wname]
    f64 = lambda t: t.float().numpy().astype(np.float64)
    a = OQ.quant_128x128(f64(synth.expert_weights(wl, "w13", e))[None])
    b = OQ.quant_128x128(f64(synth.expert_weights(wl, "w2", e))[None])
    return a[0][0], a[1][0], b[0][0], b[1][0]


def cpu_baseline(Ts):
    """The oracle's training step on the host, for the first Ts tokens of the
    headline workload and all its local experts.  Must run before the GPU is
    initialised (the setup forks a process pool)."""
    from concurrent.futures import ProcessPoolExecutor
    from moe_expert_layer_r3_amd import synth
    from oracle import layer as OL, routing as OR

    wl = synth.WORKLOADS["train"]
    ncores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    with ProcessPoolExecutor(min(ncores, 16, wl.L)) as ex:
        parts = list(ex.map(_oracle_expert_weights, [(wl.name, e) for e in range(wl.L)]))
    wq = ((np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])),
          (np.stack([p[2] for p in parts]), np.stack([p[3] for p in parts])))
    del parts
    setup_s = time.perf_counter() - t0
    lg = synth.logits(wl, T=Ts)
    x = synth.x(wl, T=Ts).float().numpy().astype(np.float64)
    dy = synth.dy(wl, T=Ts).float().numpy().astype(np.float64)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = ncores
    t1 = time.perf_counter()
    ids, w = OR.topk(lg, wl.k)
    fw = OL.forward(x, ids, w, wl.e0, wl.L, wq)
    t2 = time.perf_counter()
    OL.backward(fw, dy, ids, w, wl.E, wq)
    t3 = time.perf_counter()
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {
        "value": Ts / (t3 - t1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"train workload, tokens 0-{Ts - 1} ({int(fw['counts'].sum())} local pairs) through the whole "
                   f"training step over all {wl.L} local experts: top-k, permutation, forward, backward with "
                   f"both wgrad products and the gate backward, timed as run ({t3 - t1:.1f} s: forward "
                   f"{t2 - t1:.1f} s, backward {t3 - t2:.1f} s), no extrapolation; the oracle's 128x128 weight "
                   f"quantisation ran before, untimed ({setup_s:.1f} s in a process pool). Much of the "
                   f"backward's time is per-step work that does not scale with tokens (bf16 rounding of the fp64 "
                   f"weight gradients), so the rate at T={wl.T} would be higher."),
        "cpu_model": model,
        "host_cores": ncores,
        "seconds": t3 - t1,
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the expert-parallel exchange across GPUs is not part of it", file=sys.stderr)
        sys.exit(2)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_tokens)          # before any GPU use (the setup forks)
        print(f"# cpu baseline done ({cpu['seconds']:.1f} s)", file=sys.stderr, flush=True)
    from moe_expert_layer_r3_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS["train"]
    head = train_leg(args.steps, args.warmup, dev)
    print("# headline training step done", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate, bf16 activations)",
        "data": "synthetic (seeded normals; random-init N(0,0.02) expert weights)",
        "config": {"workload": head["workload"], "T": wl.T, "d": wl.d, "f": wl.f, "E": wl.E,
                   "local_experts": wl.L, "top_k": wl.k, "local_pairs": head["local_pairs"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "gemm_tflops": head["gemm_tflops"],
        "gemm_mfma_frac": head["gemm_mfma_frac"],
        "ms_per_step_eager": head["ms_per_step_eager"],
        "ms_per_step_excl_weight_quant": head["ms_per_step_excl_weight_quant"],
        "kernel_ms": head["kernel_ms"],
        "gemms": head["gemms"],
        "input_sets": head["input_sets"],
    }
    if cpu is None:
        del out["cpu_baseline"]
    legs = [] if args.legs == "none" else [s for s in args.legs.split(",") if s]
    out["legs"] = {}
    for leg in legs:
        if leg in ("ep8", "hotspot"):
            r = forward_leg(synth.WORKLOADS[leg], args.steps, args.warmup, dev)
            r["workload"] = {"ep8": "ep8: T=8192 share of a 256-expert top-8 layer, forward",
                             "hotspot": "hotspot: ep8 shape, logits biased -1.2 ln(e+1) (expert 0 hottest), "
                                        "forward"}[leg]
        elif leg == "pow2":
            r = forward_leg(synth.WORKLOADS["ep8"], args.steps, args.warmup, dev, pow2=True)
            r["workload"] = ("ep8 forward with power-of-two (UE8M0) tile scales applied by the block-scaled MFMA "
                             "(a variant; the other legs use fp32 scales)")
        elif leg == "mxfp4":
            r = forward_leg(synth.WORKLOADS["ep8"], args.steps, args.warmup, dev, mxfp4=True)
            r["workload"] = ("ep8 forward with MXFP4 expert weights (E2M1, E8M0 scale per 32 values) and "
                             "power-of-two FP8 activations (a variant)")
        elif leg == "train_pow2":
            r = train_leg(args.steps, args.warmup, dev, pow2=True)
        elif leg == "train_mxfp4":
            r = train_leg(args.steps, args.warmup, dev, mxfp4=True)
        elif leg == "replay":
            r = replay_leg(args.replay_passes, dev)
        else:
            raise SystemExit(f"unknown leg {leg}")
        out["legs"][leg] = r
        print(f"# leg {leg} done", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
