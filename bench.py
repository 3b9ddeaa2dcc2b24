"""Benchmark of the MoE expert layer on one MI355X.

One step = one forward pass of the layer on the EP=8 share of a 256-expert top-8
layer (T=8192 tokens, d=7168, f=2048 SwiGLU, local experts 0-31): top-k routing,
the expert-grouped permutation with fused 1x128 FP8 quantisation, grouped GEMM1
with the fused SwiGLU + quantisation epilogue, grouped GEMM2, weighted combine.
Weights are quantised once (static weights) before the timed region; that cost
is reported separately.  Inputs are seeded synthetic tensors already resident in
HBM when timing starts.

Prints one JSON line (rank 0).  Besides the throughput it reports the roofline
fraction of the dominant kernel (grouped GEMM1, HBM-bound at this shape) from
HIP events recorded on the launch stream, and the oracle's throughput on the
host cores (a bounded sample: all tokens routed and permuted, expert work for
2 of the 32 local experts, extrapolated linearly in the number of experts)."""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ep8", choices=["ep8", "hotspot"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def gemm_algorithmic(P, L, d, f):
    """Algorithmic FLOPs and HBM bytes of the two grouped GEMMs for P local pairs."""
    g1_flops = 2.0 * P * d * (2 * f)
    g2_flops = 2.0 * P * f * d
    g1_bytes = (L * 2 * f * d + L * (2 * f // 128) * (d // 128) * 4     # W13 codes + scales
                + P * d + P * (d // 128) * 4                             # Xq + scales
                + P * f + P * (f // 128) * 4)                            # hq + scales
    g2_bytes = (L * d * f + L * (d // 128) * (f // 128) * 4
                + P * f + P * (f // 128) * 4
                + P * d * 2)                                             # Y bf16
    return g1_flops, g1_bytes, g2_flops, g2_bytes


def measured_traffic(workload):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source changed since then."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"gemm1_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(here, "moe_expert_layer_r3_amd", "csrc")
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.hpp"):
        h.update(open(os.path.join(src, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def cpu_baseline(wl, lg, x_bf16, W13, W2):
    """The oracle on the host: routing + permutation for all tokens, expert work
    (gather, quantise, GEMMs, SwiGLU, combine) for 2 of the L local experts,
    extrapolated to L experts."""
    from oracle import blockfp8 as OQ, dispatch as OD, gemm as OG, layer as OL, routing as OR
    from oracle.numerics import bf16, f32
    Ls = 2
    xs = x_bf16.float().numpy().astype(np.float64)
    w13 = W13[:Ls].float().numpy().astype(np.float64)
    w2 = W2[:Ls].float().numpy().astype(np.float64)
    wq13 = OQ.quant_128x128(w13)
    wq2 = OQ.quant_128x128(w2)
    t0 = time.perf_counter()
    ids, w = OR.topk(lg, wl.k)
    c, o, rp, pr = OD.permute_index(ids, wl.e0, wl.L)
    t1 = time.perf_counter()
    # expert part for experts 0..Ls-1 (their rows only)
    c2, o2, rp2, pr2 = OD.permute_index(ids, wl.e0, Ls)
    Xp = OD.gather_rows(xs, rp2, wl.k)
    Xq, Xs = OQ.quant_1x128(Xp)
    GU = OG.grouped_forward(Xq, Xs, c2, o2, wq13[0], wq13[1])
    h = f32(OL.silu(f32(GU[:, :wl.f])) * f32(GU[:, wl.f:]))
    hq, hs = OQ.quant_1x128(h)
    Y = bf16(OG.grouped_forward(hq, hs, c2, o2, wq2[0], wq2[1]))
    OD.combine(Y, pr2, w)
    t2 = time.perf_counter()
    est = (t1 - t0) + (t2 - t1) * (wl.L / Ls)
    return {
        "value": wl.T / est,
        "unit": "tokens/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{wl.name} workload: routing and permutation of all {wl.T} tokens timed "
                   f"({t1 - t0:.2f} s); expert work for {Ls} of {wl.L} local experts timed "
                   f"({t2 - t1:.2f} s) and scaled x{wl.L // Ls}; weight quantisation excluded "
                   f"(static weights, as on the GPU)"),
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
    from moe_expert_layer_r3_amd import synth
    from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lg = synth.logits(wl)
    x = synth.x(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    lg_d = torch.from_numpy(lg).to(dev)
    x_d = x.to(dev)
    W13_d, W2_d = W13.to(dev), W2.to(dev)

    # weight quantisation (once per weight version), timed on its own
    wts = quantize_weights(W13_d, W2_d)
    torch.cuda.synchronize()
    qe0, qe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qe0.record()
    for _ in range(3):
        wts = quantize_weights(W13_d, W2_d)
    qe1.record()
    torch.cuda.synchronize()
    wquant_ms = qe0.elapsed_time(qe1) / 3
    del W13_d, W2_d
    torch.cuda.empty_cache()

    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=dev)
    for _ in range(args.warmup):
        plan.forward(x_d, lg_d, wts)
    torch.cuda.synchronize()

    names = ["route", "permute", "gemm1", "gemm2", "combine"]
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        plan.forward(x_d, lg_d, wts, events={n: ev[n][s] for n in names})
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}

    counts = plan.counts.cpu().numpy()
    P = int(counts.sum())
    g1f, g1b, g2f, g2b = gemm_algorithmic(P, wl.L, wl.d, wl.f)
    g1_s, g2_s = kern_ms["gemm1"] * 1e-3, kern_ms["gemm2"] * 1e-3
    ach_gbs = g1b / g1_s / 1e9
    gemm_tflops = (g1f + g2f) / (g1_s + g2_s) / 1e12

    out = {
        "metric": "MoE-layer tokens/s + FP8 grouped-GEMM TFLOP/s (% of MFMA peak)",
        "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate, bf16 activations)",
        "data": "synthetic (seeded normals; random-init N(0,0.02) expert weights)",
        "config": {"workload": f"{wl.name}: one EP=8 share of a 256-expert top-8 MoE layer forward",
                   "T": wl.T, "d": wl.d, "f": wl.f, "E": wl.E, "local_experts": wl.L, "top_k": wl.k,
                   "local_pairs": P},
        "roofline": {"bound": "hbm", "kernel": "grouped GEMM1 + SwiGLU + quant (gemm_fp8_kernel<256,1>)",
                     "achieved": ach_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(wl.name)},
        "gemm_tflops": gemm_tflops,
        "gemm_mfma_frac": gemm_tflops / FP8_PEAK_TFLOPS,
        "kernel_ms": kern_ms,
        "weight_quant_ms": wquant_ms,
        "expert_counts": {"max": int(counts.max()), "mean": float(counts.mean()), "min": int(counts.min())},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, lg, x, W13, W2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
