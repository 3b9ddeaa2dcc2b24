"""GPU parity of the power-of-two (UE8M0) scale variant of the forward path,
through the C ABI, against the oracle's pow2 chain.

FP8 codes and scales are bit-exact (the scale is an exponent choice and every
v * 2^-e is exact in fp32); GEMM outputs hold the same bounds as the fp32-scale
path: ACC_TOL on raw accumulators, 2e-3 relative Frobenius on bf16 outputs."""

import numpy as np
import pytest
import torch

from oracle import blockfp8 as OQ
from oracle import dispatch as OD
from oracle import gemm as OG
from oracle import layer as OL
from oracle import routing as OR
from oracle.numerics import bf16 as obf16, f32 as of32
from moe_expert_layer_r3_amd import ops, synth
from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights
from gpu_util import DEV, bf16_tensor, gpu, ids_for_counts, np64, npi, rel_fro, say
import layer_checks as LC

pytestmark = pytest.mark.gpu
TOL = 2e-3
ACC_TOL = 1e-4


def _edge_rows(rng, rows, cols):
    """Rows spanning many binades, plus tiles whose amax sits exactly on, just
    below and just above 448 * 2^k (the boundaries of the exponent choice)."""
    x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, 1)))
    x[5] = 0.0
    x[6, :128] = 2.0 ** -130
    x[7, :128] = rng.uniform(-1, 1, 128)
    x[7, 9] = 448.0 * 2.0 ** -3                      # a = 448 * 2^k: s = 2^k
    x[8, :128] = rng.uniform(-1, 1, 128)
    x[8, 0] = 448.0 * 2.0 ** 4 * (1 + 2.0 ** -7)     # just above: next exponent (bf16 ulp)
    x[9, :128] = rng.uniform(-1, 1, 128)
    x[9, 0] = -448.0 * 2.0 ** -10 * (1 - 2.0 ** -8)  # just below, negative
    return x


def test_quant_1x128_pow2_bf16_and_f32():
    rng = np.random.default_rng(20)
    xb = obf16(_edge_rows(rng, 301, 512))
    say("pow2 quant 1x128 bf16 [301, 512]")
    q, s = ops.quant_fp8(bf16_tensor(xb), pow2=True)
    rq, rs = OQ.quant_1x128(xb, pow2=True)
    assert np.array_equal(npi(q), rq)
    assert np.array_equal(npi(s).astype(np.float64), rs)
    sv = npi(s)
    assert np.all(np.frexp(sv)[0] == 0.5)            # every scale is a power of two
    xf = of32(_edge_rows(rng, 77, 384))
    say("pow2 quant 1x128 fp32 [77, 384]")
    q, s = ops.quant_fp8(gpu(xf.astype(np.float32)), pow2=True)
    rq, rs = OQ.quant_1x128(xf, pow2=True)
    assert np.array_equal(npi(q), rq)
    assert np.array_equal(npi(s).astype(np.float64), rs)


def test_quant_128x128_pow2_and_transpose():
    rng = np.random.default_rng(21)
    w = rng.standard_normal((3, 256, 384)) * 0.02
    w[1, :128, 128:256] *= 1000.0
    w[2, 128:, :128] = 0.0
    w[0, 0, 0] = 448.0 * 2.0 ** -6
    w = obf16(w)
    say("pow2 quant 128x128 [3, 256, 384] + transpose")
    q, s, qT, sT = ops.quant_fp8(bf16_tensor(w), tile=ops.TILE_128x128, transpose=True, pow2=True)
    rq, rs = OQ.quant_128x128(w, pow2=True)
    assert np.array_equal(npi(q), rq)
    assert np.array_equal(npi(s).astype(np.float64), rs)
    assert np.array_equal(npi(qT), np.swapaxes(rq, 1, 2))
    assert np.array_equal(npi(sT).astype(np.float64), np.swapaxes(rs, 1, 2))


def test_permute_gather_pow2():
    rng = np.random.default_rng(22)
    ids = ids_for_counts([0, 1, 127, 128, 129, 0, 300, 5], k=8, E=64, e0=8, rng=rng)
    x = obf16(_edge_rows(rng, ids.shape[0], 384))
    say(f"pow2 permute gather T={ids.shape[0]} d=384")
    res = ops.permute(gpu(ids), 8, 8, x=bf16_tensor(x), pow2=True)
    c, o, rp, pr = OD.permute_index(ids, 8, 8)
    n = int(o[-1])
    assert np.array_equal(npi(res["row_pair"])[:n], rp)
    real = rp >= 0
    xq, xs = OQ.quant_1x128(x, pow2=True)
    assert np.array_equal(npi(res["xq"])[:n][real], xq[rp[real] // 8])
    assert np.array_equal(npi(res["xq_s"]).T[:n][real].astype(np.float64), xs[rp[real] // 8])


def _problem(counts, K, N, seed, e0=0, E=64, k=8):
    rng = np.random.default_rng(seed)
    L = len(counts)
    ids = ids_for_counts(counts, k=k, E=E, e0=e0, rng=rng)
    x = obf16(rng.standard_normal((ids.shape[0], K)) * np.exp2(rng.integers(-8, 8, (ids.shape[0], 1))))
    res = ops.permute(gpu(ids), e0, L, x=bf16_tensor(x), pow2=True)
    W = obf16(rng.standard_normal((L, N, K)) * 0.02)
    W[0, :128] *= 50.0
    wq, ws = ops.quant_fp8(bf16_tensor(W), tile=ops.TILE_128x128, pow2=True)
    return res, wq, ws


def _real_rows(res):
    o, c = npi(res["offsets"]), npi(res["counts"])
    return np.concatenate([np.arange(o[e], o[e] + c[e]) for e in range(len(c))]).astype(np.int64)


@pytest.mark.parametrize("tile128", [False, True])
@pytest.mark.parametrize("counts,K,N", [([0, 1, 130, 300], 256, 512), ([128, 256, 5, 0, 77, 129], 384, 256),
                                        ([40], 128, 128), ([200, 3], 640, 384)])
def test_gemm_store_pow2(counts, K, N, tile128):
    res, wq, ws = _problem(counts, K, N, seed=K + N + 100)
    say(f"pow2 gemm STORE counts={counts} K={K} N={N} tile128={tile128}")
    args = (res["xq"], res["xq_s"], wq, ws, res["counts"], res["offsets"])
    acc = ops.grouped_gemm(*args, ops.EPI_STORE_F32, pow2=True, tile128=tile128)
    y = ops.grouped_gemm(*args, ops.EPI_STORE_BF16, pow2=True, tile128=tile128)
    c, o = npi(res["counts"]), npi(res["offsets"])
    ref = OG.grouped_forward(npi(res["xq"]), npi(res["xq_s"]).T, c, o, npi(wq), npi(ws))
    rows = _real_rows(res)
    assert rel_fro(np64(acc)[rows], ref[rows]) <= ACC_TOL
    assert rel_fro(np64(y)[rows], obf16(ref[rows])) <= TOL
    # the fp32-scale kernel on the same (power-of-two) scales sums the same terms
    acc32 = ops.grouped_gemm(*args, ops.EPI_STORE_F32, tile128=tile128)
    assert rel_fro(np64(acc)[rows], np64(acc32)[rows]) <= ACC_TOL


@pytest.mark.parametrize("tile128", [False, True])
@pytest.mark.parametrize("counts,K,f", [([0, 1, 130, 300], 256, 256), ([129, 64], 384, 384), ([256], 128, 128)])
def test_gemm_swiglu_pow2(counts, K, f, tile128):
    res, wq, ws = _problem(counts, K, 2 * f, seed=K + f + 101)
    say(f"pow2 gemm SWIGLU counts={counts} K={K} f={f} tile128={tile128}")
    args = (res["xq"], res["xq_s"], wq, ws, res["counts"], res["offsets"])
    h32 = ops.grouped_gemm(*args, ops.EPI_SWIGLU_F32, pow2=True, tile128=tile128)
    hq, hs = ops.grouped_gemm(*args, ops.EPI_SWIGLU_Q8, pow2=True, tile128=tile128)
    hq2, hs2, gu = ops.grouped_gemm(*args, ops.EPI_SWIGLU_Q8_SAVE, pow2=True, tile128=tile128)
    c, o = npi(res["counts"]), npi(res["offsets"])
    GU = OG.grouped_forward(npi(res["xq"]), npi(res["xq_s"]).T, c, o, npi(wq), npi(ws))
    f_ = GU.shape[1] // 2
    h_ref = OL.silu(of32(GU[:, :f_])) * of32(GU[:, f_:])
    rows = _real_rows(res)
    assert rel_fro(np64(h32)[rows], h_ref[rows]) <= ACC_TOL
    qref, sref = OQ.quant_1x128(np64(h32)[rows], pow2=True)
    assert np.array_equal(npi(hq)[rows], qref)
    assert np.array_equal(npi(hs).T[rows].astype(np.float64), sref)
    assert np.array_equal(npi(hq2)[rows], npi(hq)[rows]) and np.array_equal(npi(hs2).T[rows], npi(hs).T[rows])
    assert rel_fro(np64(gu)[rows], obf16(GU[rows])) <= TOL


def _plan_forward(wl, pow2):
    lg = synth.logits(wl)
    x = synth.x(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    wts = quantize_weights(W13.to(DEV), W2.to(DEV), pow2=pow2)
    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=DEV, pow2=pow2)
    y = plan.forward(x.to(DEV), gpu(lg), wts)
    torch.cuda.synchronize()
    return lg, x, W13, W2, wts, plan, y


def test_layer_tiny_forward_pow2():
    wl = synth.WORKLOADS["tiny"]
    say("pow2 tiny layer forward through ForwardPlan")
    lg, x, W13, W2, wts, plan, y = _plan_forward(wl, True)
    ids, w = OR.topk(lg, wl.k)
    assert np.array_equal(npi(plan.ids), ids)
    wq = OL.quantize_weights(np64(W13), np64(W2), pow2=True)
    assert np.array_equal(npi(wts["w13q"]), wq[0][0]) and np.array_equal(npi(wts["w2q"]), wq[1][0])
    assert np.array_equal(npi(wts["w13s"]).astype(np.float64), wq[0][1])
    fw = OL.forward(np64(x), ids, w, wl.e0, wl.L, wq, pow2=True)
    e = rel_fro(np64(y), fw["y"])
    say("pow2 tiny layer rel err", e)
    assert e <= TOL


def test_layer_ep8_full_size_sampled_pow2():
    """The full EP=8 share (T=8192, d=7168, f=2048, 32 of 256 experts, top-8)
    through ForwardPlan with power-of-two scales, as the benchmark runs it;
    sampled rows of two experts and of the combine against the oracle."""
    LC.full_size_forward_check(synth.WORKLOADS["ep8"], experts=(0, 17, 31), pow2=True)
