"""GPU parity of the MXFP4-weight forward (E2M1 codes with an E8M0 scale per 32
values, FP8 activations with power-of-two 1x128 scales) against the oracle,
through the C ABI.

Codes and scale bytes are bit-exact; GEMM outputs hold the bounds of the FP8
path (1e-4 on fp32 accumulators, 2e-3 relative Frobenius on bf16 outputs and
the layer output) against the oracle's fp64 products over the same operands."""

import numpy as np
import pytest
import torch

from oracle import blockfp8 as OQ
from oracle import layer as OL
from oracle import mxfp4 as MX
from oracle import routing as OR
from oracle.numerics import bf16 as obf16, f32 as of32
from moe_expert_layer_r3_amd import ops, synth
from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights
from gpu_util import DEV, bf16_tensor, gpu, ids_for_counts, np64, npi, rel_fro, say
import layer_checks as LC

pytestmark = pytest.mark.gpu
TOL = 2e-3
ACC_TOL = 1e-4


def test_quant_mxfp4_bit_exact():
    rng = np.random.default_rng(60)
    w = rng.standard_normal((3, 70, 384)) * np.exp2(rng.integers(-30, 30, (3, 70, 1)))
    w[0, 0, :32] = 0.0                                  # zero block
    w[0, 1, :32] = 2.0 ** -133                          # subnormal block
    w[0, 2, :32] = 0.5
    w[0, 2, 7] = 6.0 * 2.0 ** -4                        # amax = 6 * 2^k: exact
    w[0, 3, :32] = -0.25
    w[0, 3, 9] = -7.5 * 2.0 ** 3                        # saturates
    w[0, 4, 32:64] = -0.0
    w[1, 5, :] = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]), 48)  # ties at X = 1
    w = obf16(w)
    say("mxfp4 quant [3, 70, 384]")
    q, s = ops.quant_mxfp4(bf16_tensor(w))
    codes, sc = MX.quant_mx(w)
    assert np.array_equal(ops.mx_scales_rows(s), sc)
    assert np.array_equal(ops.mx_codes_rows(q), MX.pack(codes))


def _real_rows(res):
    o, c = npi(res["offsets"]), npi(res["counts"])
    return np.concatenate([np.arange(o[e], o[e] + c[e]) for e in range(len(c))]).astype(np.int64)


def _problem(counts, K, N, seed, e0=0, E=64, k=8):
    rng = np.random.default_rng(seed)
    L = len(counts)
    ids = ids_for_counts(counts, k=k, E=E, e0=e0, rng=rng)
    x = obf16(rng.standard_normal((ids.shape[0], K)) * np.exp2(rng.integers(-6, 6, (ids.shape[0], 1))))
    res = ops.permute(gpu(ids), e0, L, x=bf16_tensor(x), pow2=True)
    W = obf16(rng.standard_normal((L, N, K)) * 0.02 * np.exp2(rng.integers(-3, 3, (L, N, 1))))
    W[0, :64] *= 40.0
    q, s = ops.quant_mxfp4(bf16_tensor(W))
    return res, q, s


def _ref(res, q, s):
    c, o = npi(res["counts"]), npi(res["offsets"])
    return MX.grouped_forward(npi(res["xq"]), npi(res["xq_s"]).T, c, o, MX.unpack(ops.mx_codes_rows(q)), ops.mx_scales_rows(s))


@pytest.mark.parametrize("tile128", [False, True])
@pytest.mark.parametrize("counts,K,N", [([0, 1, 130, 300], 256, 512), ([128, 256, 5, 0, 77, 129], 384, 256),
                                        ([40], 128, 128), ([200, 3], 640, 384)])
def test_gemm_store_mxfp4(counts, K, N, tile128):
    res, q, s = _problem(counts, K, N, seed=K + N + 200)
    say(f"mxfp4 gemm STORE counts={counts} K={K} N={N} tile128={tile128}")
    args = (res["xq"], res["xq_s"], q, s, res["counts"], res["offsets"])
    acc = ops.grouped_gemm(*args, ops.EPI_STORE_F32, mxfp4=True, tile128=tile128)
    y = ops.grouped_gemm(*args, ops.EPI_STORE_BF16, mxfp4=True, tile128=tile128)
    ref = _ref(res, q, s)
    rows = _real_rows(res)
    assert rel_fro(np64(acc)[rows], ref[rows]) <= ACC_TOL
    assert rel_fro(np64(y)[rows], obf16(ref[rows])) <= TOL


@pytest.mark.parametrize("tile128", [False, True])
@pytest.mark.parametrize("counts,K,f", [([0, 1, 130, 300], 256, 256), ([129, 64], 384, 384), ([256], 128, 128)])
def test_gemm_swiglu_mxfp4(counts, K, f, tile128):
    res, q, s = _problem(counts, K, 2 * f, seed=K + f + 201)
    say(f"mxfp4 gemm SWIGLU counts={counts} K={K} f={f} tile128={tile128}")
    args = (res["xq"], res["xq_s"], q, s, res["counts"], res["offsets"])
    h32 = ops.grouped_gemm(*args, ops.EPI_SWIGLU_F32, mxfp4=True, tile128=tile128)
    hq, hs = ops.grouped_gemm(*args, ops.EPI_SWIGLU_Q8, mxfp4=True, tile128=tile128)
    GU = _ref(res, q, s)
    h_ref = OL.silu(of32(GU[:, :f])) * of32(GU[:, f:])
    rows = _real_rows(res)
    assert rel_fro(np64(h32)[rows], h_ref[rows]) <= ACC_TOL
    qref, sref = OQ.quant_1x128(np64(h32)[rows], pow2=True)
    assert np.array_equal(npi(hq)[rows], qref)
    assert np.array_equal(npi(hs).T[rows].astype(np.float64), sref)


def _plan_forward(wl):
    lg = synth.logits(wl)
    x = synth.x(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    wts = quantize_weights(W13.to(DEV), W2.to(DEV), mxfp4=True)
    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=DEV, mxfp4=True)
    y = plan.forward(x.to(DEV), gpu(lg), wts)
    torch.cuda.synchronize()
    return lg, x, W13, W2, wts, plan, y


def test_layer_tiny_forward_mxfp4():
    wl = synth.WORKLOADS["tiny"]
    say("mxfp4 tiny layer forward through ForwardPlan")
    lg, x, W13, W2, wts, plan, y = _plan_forward(wl)
    ids, w = OR.topk(lg, wl.k)
    assert np.array_equal(npi(plan.ids), ids)
    wq = OL.quantize_weights(np64(W13), np64(W2), mx=True)
    assert np.array_equal(MX.unpack(ops.mx_codes_rows(wts["w13q"])), wq[0][0])
    assert np.array_equal(ops.mx_scales_rows(wts["w13s"]), wq[0][1])
    assert np.array_equal(MX.unpack(ops.mx_codes_rows(wts["w2q"])), wq[1][0])
    assert np.array_equal(ops.mx_scales_rows(wts["w2s"]), wq[1][1])
    fw = OL.forward(np64(x), ids, w, wl.e0, wl.L, wq, mx=True)
    e = rel_fro(np64(y), fw["y"])
    say("mxfp4 tiny layer rel err", e)
    assert e <= TOL


def test_layer_ep8_full_size_sampled_mxfp4():
    """The EP=8 share (T=8192, d=7168, f=2048, 32 of 256 experts, top-8) with
    MXFP4 weights through ForwardPlan, as the benchmark runs it; sampled rows
    of two experts and of the combine against the oracle."""
    LC.full_size_forward_check(synth.WORKLOADS["ep8"], experts=(0, 17, 31), mxfp4=True)


# ------------------------------------------------------------------ training with MXFP4 weights

def test_quant_mxfp4_transpose_bit_exact():
    rng = np.random.default_rng(61)
    w = rng.standard_normal((3, 256, 384)) * np.exp2(rng.integers(-20, 20, (3, 256, 1)))
    w[0, :32, 5] = 0.0                                 # zero column block
    w[1, 64:96, 7] = 2.0 ** -133                       # subnormal column block
    w[2, 128:160, 9] = -7.5 * 2.0 ** 2                 # saturating column block
    w = obf16(w)
    say("mxfp4 quant with transpose [3, 256, 384]")
    q, s, qT, sT = ops.quant_mxfp4(bf16_tensor(w), transpose=True)
    q1, s1 = ops.quant_mxfp4(bf16_tensor(w))
    assert torch.equal(q, q1) and torch.equal(s, s1)    # the fused pass writes the same forward codes
    codes, sc = MX.quant_mx(np.swapaxes(w, 1, 2))
    assert np.array_equal(ops.mx_scales_rows(sT), sc)
    assert np.array_equal(ops.mx_codes_rows(qT), MX.pack(codes))


@pytest.mark.parametrize("counts,K,N", [([0, 1, 130, 300], 256, 512), ([77, 128], 384, 256)])
def test_gemm_dgrad_mxfp4(counts, K, N):
    """acc[r] = dY[r] @ W[e] with W [L, K, N] in its forward [out, in] layout:
    the GEMM reads the transposed MXFP4 copy (blocks along K)."""
    rng = np.random.default_rng(K + N + 300)
    L = len(counts)
    ids = ids_for_counts(counts, k=4, E=32, e0=0, rng=rng)
    res = ops.permute(gpu(ids), 0, L)
    rcap = res["row_cap"]
    A = obf16(rng.standard_normal((rcap, K)))
    aq, as_ = ops.quant_fp8(bf16_tensor(A), pow2=True)
    W = obf16(rng.standard_normal((L, K, N)) * 0.02)
    W[0, :128] *= 30.0
    _, _, qT, sT = ops.quant_mxfp4(bf16_tensor(W), transpose=True)
    say(f"mxfp4 gemm dgrad counts={counts} K={K} N={N}")
    acc = ops.grouped_gemm(aq, as_.t().contiguous(), qT, sT, res["counts"], res["offsets"], ops.EPI_STORE_F32,
                           mxfp4=True)
    c, o = npi(res["counts"]), npi(res["offsets"])
    ref = MX.grouped_forward(npi(aq), npi(as_), c, o, MX.unpack(ops.mx_codes_rows(qT)), ops.mx_scales_rows(sT))
    assert rel_fro(np64(acc)[_real_rows(res)], ref[_real_rows(res)]) <= ACC_TOL


def _train(wl):
    from moe_expert_layer_r3_amd.layer import TrainPlan
    lg = synth.logits(wl)
    x = synth.x(wl)
    dy = synth.dy(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    wts = quantize_weights(W13.to(DEV), W2.to(DEV), transpose=True, mxfp4=True)
    plan = TrainPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, e0=wl.e0, device=DEV, mxfp4=True)
    plan.forward(x.to(DEV), gpu(lg), wts)
    plan.backward(x.to(DEV), dy.to(DEV), wts)
    torch.cuda.synchronize()
    return lg, x, dy, W13, W2, wts, plan


def test_layer_tiny_train_mxfp4():
    wl = synth.WORKLOADS["tiny"]
    say("mxfp4 tiny layer forward + backward")
    lg, x, dy, W13, W2, wts, plan = _train(wl)
    ids, w = OR.topk(lg, wl.k)
    wq = OL.quantize_weights(np64(W13), np64(W2), mx=True)
    assert np.array_equal(MX.unpack(ops.mx_codes_rows(wts["w13qT"])), wq[0][2])
    assert np.array_equal(ops.mx_scales_rows(wts["w2sT"]), wq[1][3])
    fw = OL.forward(np64(x), ids, w, wl.e0, wl.L, wq, mx=True)
    bw = OL.backward(fw, np64(dy), ids, w, wl.E, wq, mx=True)
    # as for the FP8 chain: the two chains take their FP8 rounding decisions
    # on values that differ by fp32 rounding, so 1e-2 bounds the end result
    for name, got, ref in (("y", plan.y, fw["y"]), ("dx", plan.dx, bw["dx"]), ("dW2", plan.dW2, bw["dW2"]),
                           ("dW13", plan.dW13, bw["dW13"]), ("d_logits", plan.d_logits, bw["d_logits"])):
        err = rel_fro(np64(got), ref)
        say(f"mxfp4 tiny chain {name}: rel err {err:.2e}")
        assert err <= 1e-2, name


def test_layer_train_full_size_sampled_mxfp4():
    """T=16384 training step with MXFP4 weights through TrainPlan, as the
    benchmark runs it: both dgrad products on sampled rows of two experts,
    against the oracle over the GPU's own operands."""
    wl = synth.WORKLOADS["train"]
    say("mxfp4 train: GPU forward + backward")
    lg, x, dy, W13, W2, wts, plan = _train(wl)
    c, o = npi(plan.counts), npi(plan.offsets)
    for e in (0, 21):
        rows = np.arange(o[e], o[e] + c[e])[:: max(1, c[e] // 16)]
        idx = torch.as_tensor(rows, device=DEV)
        w2T = MX.unpack(ops.mx_codes_rows(wts["w2qT"][e:e + 1])[0]), ops.mx_scales_rows(wts["w2sT"][e:e + 1])[0]
        c2, s2 = MX.quant_mx(np64(W2[e]).T)
        assert np.array_equal(w2T[0], c2) and np.array_equal(w2T[1], s2)
        dH = MX.matmul(npi(plan.dyq[idx]), np64(plan.dyq_s.t()[idx]), *w2T)
        assert rel_fro(np64(plan.dH[idx]), dH) <= ACC_TOL
        w13T = MX.unpack(ops.mx_codes_rows(wts["w13qT"][e:e + 1])[0]), ops.mx_scales_rows(wts["w13sT"][e:e + 1])[0]
        dX = MX.matmul(npi(plan.sb["dgu_q"][idx]), np64(plan.sb["dgu_s"].t()[idx]), *w13T)
        assert rel_fro(np64(plan.dX[idx]), obf16(dX)) <= TOL
    say("mxfp4 train sampled dgrad parity ok")
