"""GPU parity of the training backward against the oracle, through the C ABI.

Each stage is checked on the operands the GPU itself produced upstream, so that
the bar of the forward tests applies unchanged: FP8 codes and scales bit-exact
against the oracle's quantiser applied to the GPU's own fp32 values; GEMM
outputs within 2e-3 relative Frobenius of the oracle's fp64 accumulation over
the identical FP8 operands (raw fp32 accumulators within 1e-4)."""

import numpy as np
import pytest
import torch

from oracle import blockfp8 as OQ
from oracle import dispatch as OD
from oracle import gemm as OG
from oracle import layer as OL
from oracle import routing as OR
from oracle.numerics import bf16 as obf16, f32 as of32
from moe_expert_layer_r3_amd import layer as ML
from moe_expert_layer_r3_amd import ops, synth
from gpu_util import DEV, bf16_tensor, gpu, ids_for_counts, np64, npi, rel_fro, say
import layer_checks as LC

pytestmark = pytest.mark.gpu
TOL = 2e-3
ACC_TOL = 1e-4


def _perm(counts, k, E, e0, seed):
    rng = np.random.default_rng(seed)
    ids = ids_for_counts(counts, k=k, E=E, e0=e0, rng=rng)
    res = ops.permute(gpu(ids), e0, len(counts))
    c, o, rp, pr = OD.permute_index(ids, e0, len(counts))
    assert np.array_equal(npi(res["offsets"]), o)
    n = int(o[-1])
    assert np.array_equal(npi(res["row_pair"])[:n], rp)
    return ids, res, rp, rng


def _bf16_rows(rng, T, cols):
    v = rng.standard_normal((T, cols)) * np.exp2(rng.integers(-8, 8, (T, 1)))
    return obf16(v)


# ------------------------------------------------------------------ 128x1 quantisation

@pytest.mark.parametrize("weighted,pow2", [(True, False), (False, False), (True, True)])
def test_quant_rows_t(weighted, pow2):
    counts, k, E, e0 = [0, 1, 130, 300, 128], 4, 40, 3
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=21 + weighted)
    T, cols = ids.shape[0], 384
    src = _bf16_rows(rng, T, cols)
    src[7, :] = 0.0
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    say(f"quant_rows_t weighted={weighted} pow2={pow2} counts={counts}")
    rcap = res["row_cap"]
    qT, sT = ops.quant_rows_t(bf16_tensor(src), None if w is None else gpu(w), res["row_pair"], res["offsets"],
                              len(counts), rcap, k, pow2=pow2)
    n = len(rp)
    real = rp >= 0
    v = np.zeros((n, cols))
    p = rp[real]
    v[real] = src[p // k] if w is None else of32(w.reshape(-1)[p][:, None].astype(np.float64) * src[p // k])
    rq, rs = OQ.quant_128x1_t(v, real, pow2=pow2)
    assert np.array_equal(npi(ops.untile_t(qT))[:, :n], rq)
    assert np.array_equal(npi(sT)[:n // 128].T.astype(np.float64), rs)


@pytest.mark.parametrize("weighted,pow2,cols", [(False, False, 384), (True, False, 640), (False, True, 2176)])
def test_quant_rows_both(weighted, pow2, cols):
    """The grouped rows quantised 1x128 (as the permutation's gather writes xq)
    and 128x1 (as quant_rows_t writes) from one read."""
    counts, k, E, e0 = [0, 1, 130, 300, 128, 257], 4, 40, 3
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=41 + cols + weighted)
    T = ids.shape[0]
    src = _bf16_rows(rng, T, cols)
    src[5, :] = 0.0
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    say(f"quant_rows_both weighted={weighted} pow2={pow2} cols={cols}")
    rcap = res["row_cap"]
    q, qs, qT, qTs = ops.quant_rows_both(bf16_tensor(src), None if w is None else gpu(w), res["row_pair"],
                                         res["offsets"], len(counts), rcap, k, pow2=pow2)
    n = int(npi(res["offsets"])[-1])
    real = rp >= 0
    rows = np.flatnonzero(real)
    p = rp[real]
    v = np.zeros((n, cols))
    v[real] = src[p // k] if w is None else of32(w.reshape(-1)[p][:, None].astype(np.float64) * src[p // k])
    rq, rs = OQ.quant_1x128(v[real], pow2=pow2)
    assert np.array_equal(npi(q)[rows], rq)
    assert np.array_equal(npi(qs).T[rows].astype(np.float64), rs)
    tq, ts = OQ.quant_128x1_t(v, real, pow2=pow2)
    assert np.array_equal(npi(ops.untile_t(qT))[:, :n], tq)
    assert np.array_equal(npi(qTs)[:n // 128].T.astype(np.float64), ts)


# ------------------------------------------------------------------ combine backward

@pytest.mark.parametrize("pow2", [False, True])
def test_combine_backward(pow2):
    rng = np.random.default_rng(31)
    T, E, k, e0, L, d = 2000, 64, 6, 16, 16, 512
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = OR.topk(lg, k)
    res = ops.permute(gpu(ids), e0, L)
    rcap = res["row_cap"]
    Y = obf16(rng.standard_normal((rcap, d)))
    dy = _bf16_rows(rng, T, d)
    say(f"combine backward pow2={pow2}")
    dyq, dys, d_gate = ops.combine_backward(bf16_tensor(dy), bf16_tensor(Y), res["pair_row"],
                                            gpu(w.astype(np.float32)), pow2=pow2)
    pr = npi(res["pair_row"])
    rp = npi(res["row_pair"])[:int(npi(res["offsets"])[-1])]
    real = rp >= 0
    rows = np.flatnonzero(real)
    t, j = rp[real] // k, rp[real] % k
    rq, rs = OQ.quant_1x128(of32(w[t, j][:, None] * dy[t]), pow2=pow2)
    assert np.array_equal(npi(dyq)[rows], rq)
    assert np.array_equal(npi(dys).T[rows].astype(np.float64), rs)
    g = np64(d_gate)
    loc = pr >= 0
    ref = np.zeros((T, k))
    prod = dy[np.nonzero(loc)[0]] * Y[pr[loc]]
    ref[loc] = np.sum(prod, axis=1)
    bound = 1e-6 * np.sum(np.abs(prod), axis=1) + 1e-30
    assert np.all(np.abs(g[loc] - ref[loc]) <= bound)
    assert np.all(g[~loc] == 0.0)


@pytest.mark.parametrize("counts,k,d,pow2", [
    ([0, 1, 130, 300, 128, 0, 77], 6, 512, False),     # one column group, ragged segments, empty experts
    ([0, 1, 130, 300, 128, 0, 77], 6, 512, True),
    ([255, 3, 129, 0, 600], 8, 2176, False),           # 17 chunks: 5 groups, the last one chunk wide
    ([40, 0, 97], 2, 128, True),                        # one chunk
])
def test_combine_backward_rows(counts, k, d, pow2):
    """dY = fp32(w * dy) on the grouped rows quantised 1x128 and 128x1 from one
    pass, and d_gate / d_logits from its per-group partials."""
    E, e0 = 40, 3
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=61 + d + k)
    T, L = ids.shape[0], len(counts)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    rcap = res["row_cap"]
    Y = obf16(rng.standard_normal((rcap, d)))
    dy = _bf16_rows(rng, T, d)
    dy[3, :] = 0.0
    say(f"combine backward rows counts={counts} k={k} d={d} pow2={pow2}")
    dyq, dys, dyqT, dyqT_s, part = ops.combine_backward_rows(bf16_tensor(dy), bf16_tensor(Y), gpu(w),
                                                             res["row_pair"], res["offsets"], L, rcap, k,
                                                             pow2=pow2)
    d_gate, d_logits = ops.gate_backward_parts(part, res["pair_row"], rcap, d, gpu(w), gpu(ids), E)
    n = int(npi(res["offsets"])[-1])
    real = rp >= 0
    rows = np.flatnonzero(real)
    t, j = rp[real] // k, rp[real] % k
    dY = of32(w[t, j][:, None].astype(np.float64) * dy[t])
    rq, rs = OQ.quant_1x128(dY, pow2=pow2)
    assert np.array_equal(npi(dyq)[rows], rq)
    assert np.array_equal(npi(dys).T[rows].astype(np.float64), rs)
    v = np.zeros((n, d))
    v[real] = dY
    tq, ts = OQ.quant_128x1_t(v, real, pow2=pow2)
    assert np.array_equal(npi(ops.untile_t(dyqT))[:, :n], tq)
    assert np.array_equal(npi(dyqT_s)[:n // 128].T.astype(np.float64), ts)
    pr = npi(res["pair_row"])
    loc = pr >= 0
    prod = dy[np.nonzero(loc)[0]] * Y[pr[loc]]
    g = np64(d_gate)
    bound = 1e-6 * np.sum(np.abs(prod), axis=1) + 1e-30
    assert np.all(np.abs(g[loc] - np.sum(prod, axis=1)) <= bound)
    assert np.all(g[~loc] == 0.0)
    dl = OR.gate_backward(g, w, ids, E)
    gmax = np.max(np.abs(g), axis=1, keepdims=True)
    assert np.all(np.abs(np64(d_logits) - dl) <= 1e-6 * gmax + 1e-30)


# ------------------------------------------------------------------ SwiGLU backward

def _swiglu_ref(dH, G, U):
    s = OL.sigmoid(G)
    dG = dH * U * s * (1.0 + G * (1.0 - s))
    dU = dH * G * s
    return np.concatenate([dG, dU], axis=1), G * s * U


def _tile_close(got, ref, width=128):
    """|got - ref| <= 1e-5 * (|ref| + max |ref| over the element's 1x128 tile)."""
    r = ref.reshape(ref.shape[0], -1, width)
    amax = np.max(np.abs(r), axis=2, keepdims=True)
    err = np.abs(got.reshape(r.shape) - r)
    return bool(np.all(err <= 1e-5 * (np.abs(r) + amax)))


@pytest.mark.parametrize("counts,f,pow2", [([0, 1, 130, 300], 256, False), ([128, 5], 128, False),
                                           ([257, 0, 64], 384, False), ([0, 1, 130, 300], 256, True)])
def test_swiglu_backward(counts, f, pow2):
    k, E, e0 = 2, 16, 0
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=41 + f)
    rcap = res["row_cap"]
    n = len(rp)
    real = rp >= 0
    rows = np.flatnonzero(real)
    dH = (rng.standard_normal((rcap, f)) * np.exp2(rng.integers(-6, 6, (rcap, 1)))).astype(np.float32)
    dH[~np.concatenate([real, np.zeros(rcap - n, bool)])] = np.nan   # padding rows must never be read
    GU = obf16(rng.standard_normal((rcap, 2 * f)) * 3.0)
    GU[rows[:3], :4] = [[-100.0, 100.0, 0.0, -1.25]] * 3                 # sigmoid tails, exact zero, dG ~ 0
    say(f"swiglu backward counts={counts} f={f} pow2={pow2}")
    o = ops.swiglu_backward(gpu(dH), bf16_tensor(GU), res["row_pair"], res["offsets"], len(counts), rcap,
                            inspect=True, pow2=pow2)
    dgu = np64(o["dgu"])[:n]
    h = np64(o["h"])[:n]
    ref_dgu, ref_h = _swiglu_ref(dH[:n].astype(np.float64), GU[:n, :f], GU[:n, f:])
    assert _tile_close(dgu[rows], ref_dgu[rows])
    assert _tile_close(h[rows], ref_h[rows])
    # fused quantisers, bit-exact on the GPU's own fp32 values
    dgu[~real] = 0.0
    h[~real] = 0.0
    q1, s1 = OQ.quant_1x128(dgu[rows], pow2=pow2)
    assert np.array_equal(npi(o["dgu_q"])[rows], q1)
    assert np.array_equal(npi(o["dgu_s"]).T[rows].astype(np.float64), s1)
    qt, st = OQ.quant_128x1_t(dgu, real, pow2=pow2)
    assert np.array_equal(npi(ops.untile_t(o["dgu_qT"]))[:, :n], qt)
    assert np.array_equal(npi(o["dgu_sT"])[:n // 128].T.astype(np.float64), st)
    qh, sh = OQ.quant_128x1_t(h, real, pow2=pow2)
    assert np.array_equal(npi(ops.untile_t(o["h_qT"]))[:, :n], qh)
    assert np.array_equal(npi(o["h_sT"])[:n // 128].T.astype(np.float64), sh)
    # the production call (no inspection outputs) writes the same bytes
    o2 = ops.swiglu_backward(gpu(dH), bf16_tensor(GU), res["row_pair"], res["offsets"], len(counts), rcap,
                             pow2=pow2)
    assert np.array_equal(npi(o2["dgu_q"])[rows], npi(o["dgu_q"])[rows])
    assert np.array_equal(npi(o2["dgu_s"]).T[rows], npi(o["dgu_s"]).T[rows])
    for key in ("dgu_qT", "h_qT"):
        assert np.array_equal(npi(o2[key])[:n // 128], npi(o[key])[:n // 128])


# ------------------------------------------------------------------ dgrad GEMM (transposed weights)

@pytest.mark.parametrize("kn", [False, True])
@pytest.mark.parametrize("counts,K,N,pow2", [([0, 1, 130, 300], 256, 512, False), ([77, 128], 384, 256, False),
                                             ([77, 128], 384, 256, True), ([300, 0, 5, 260], 1024, 768, True)])
def test_gemm_dgrad(counts, K, N, pow2, kn):
    """acc[r] = dY[r] @ W[e] for W [L, K, N] given in its forward [out=K, in=N]
    layout; the GEMM reads the transposed copy written by the 128x128 quantiser,
    or (kn) the forward codes and scales themselves as its [K, N] operand."""
    k, E, e0 = 4, 32, 0
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=K + N + 5)
    L = len(counts)
    rcap = res["row_cap"]
    A = obf16(rng.standard_normal((rcap, K)))
    aq, as_ = ops.quant_fp8(bf16_tensor(A), pow2=pow2)
    W = obf16(rng.standard_normal((L, K, N)) * 0.02)
    W[0, :128] *= 30.0
    wq, ws, wqT, wsT = ops.quant_fp8(bf16_tensor(W), tile=ops.TILE_128x128, transpose=True, pow2=pow2)
    say(f"gemm dgrad counts={counts} K={K} N={N} pow2={pow2}")
    # the GEMM reads activation scales K-block-major
    if kn:
        acc = ops.grouped_gemm(aq, as_.t().contiguous(), wq, ws, res["counts"], res["offsets"], ops.EPI_STORE_F32,
                               pow2=pow2, b_kn=True)
        # the bf16 store epilogue reads the same operands
        y = ops.grouped_gemm(aq, as_.t().contiguous(), wq, ws, res["counts"], res["offsets"], ops.EPI_STORE_BF16,
                             pow2=pow2, b_kn=True)
    else:
        acc = ops.grouped_gemm(aq, as_.t().contiguous(), wqT, wsT, res["counts"], res["offsets"], ops.EPI_STORE_F32,
                               pow2=pow2)
    c, o = npi(res["counts"]), npi(res["offsets"])
    ref = OG.grouped_dgrad(npi(aq), npi(as_), c, o, npi(wq), npi(ws))
    rows = np.concatenate([np.arange(o[e], o[e] + c[e]) for e in range(L)]).astype(np.int64)
    assert rel_fro(np64(acc)[rows], ref[rows]) <= ACC_TOL
    if kn:
        assert rel_fro(np64(y)[rows], obf16(ref[rows])) <= TOL


# ------------------------------------------------------------------ wgrad GEMM

def _abs_codes(q):
    """e4m3 codes of |v| (sign bit cleared)."""
    return np.asarray(q) & np.uint8(0x7F)


def _wgrad_check(got, ref, absum):
    """bf16 result against the fp64 accumulation: the Frobenius bar, and per
    element one bf16 rounding plus an accumulation error proportional to the
    sum of the absolute products (absum, the same accumulation over |codes|):
    the MFMA's error follows the terms' magnitudes, not the result's."""
    assert rel_fro(got, ref) <= TOL
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + ACC_TOL * absum
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"element {i}: got {got[i]!r} ref {ref[i]!r} |terms| {absum[i]!r}")


# the last case puts several tiles (of 1-, 2- and 3-block experts, with empty
# experts between them) into each workgroup's stream of K steps
_MANY = [(i * 37) % 300 if i % 7 else 0 for i in range(40)]


# tile128: the 128 x 256 kernel where the default would take 256 x 256 tiles
@pytest.mark.parametrize("counts,M,N,pow2,tile128", [
    ([0, 1, 130, 300], 256, 512, False, False), ([128, 256, 0, 5], 128, 128, False, False),
    ([1500], 384, 256, False, False), ([0, 0], 128, 256, False, False),
    (_MANY, 512, 1024, False, False), ([0, 1, 130, 300], 256, 512, True, False),
    ([128, 256, 0, 5], 128, 128, True, False), (_MANY, 512, 1024, True, False),
    ([0, 1, 130, 300, 700], 512, 256, False, False), ([0, 1, 130, 300, 700], 512, 256, True, False),
    ([0, 1, 130, 300], 256, 512, False, True), (_MANY, 512, 1024, False, True), (_MANY, 512, 1024, True, True),
    ([0, 1, 130, 300, 700], 384, 512, True, False),
    # 640 (expert, m-tile) units: the 128 x 256 kernels' persistent workgroups
    # take two or three each and switch units mid-stream
    (_MANY, 2048, 256, False, False), (_MANY, 1920, 256, True, False)])
def test_wgrad(counts, M, N, pow2, tile128):
    k = 2 if len(counts) <= 8 else 8
    E, e0 = max(16, len(counts) + k), 0
    ids, res, rp, rng = _perm(counts, k, E, e0, seed=M + N + len(counts))
    L = len(counts)
    rcap = res["row_cap"]
    n = len(rp)
    real = rp >= 0
    A = rng.standard_normal((n, M)) * np.exp2(rng.integers(-4, 4, (1, M)))
    B = rng.standard_normal((n, N))
    qa, sa = OQ.quant_128x1_t(A, real, pow2=pow2)
    qb, sb = OQ.quant_128x1_t(B, real, pow2=pow2)
    # rows past offsets[L] hold NaN codes and scales: the kernel must not read
    # them; scales go in token-block-major, the layout the kernel reads
    def upload(q, s):
        qf = np.full((q.shape[0], rcap), 0x7F, dtype=np.uint8)
        sf = np.full((rcap // 128, q.shape[0]), np.nan, dtype=np.float32)
        qf[:, :n] = q
        sf[:n // 128] = s.T
        return gpu(ops.tile_t(qf)), gpu(sf)
    aT, aT_s = upload(qa, sa)
    bT, bT_s = upload(qb, sb)
    say(f"wgrad counts={counts} M={M} N={N} pow2={pow2} tile128={tile128}")
    dW = ops.grouped_gemm_wgrad(aT, aT_s, bT, bT_s, res["offsets"], L, rcap, pow2=pow2, tile128=tile128)
    c, o = npi(res["counts"]), npi(res["offsets"])
    ref = OG.grouped_wgrad(qa, sa, qb, sb, c, o)
    absum = OG.grouped_wgrad(_abs_codes(qa), sa, _abs_codes(qb), sb, c, o)
    got = np64(dW)
    for e in range(L):
        if c[e] == 0:
            assert np.all(got[e] == 0.0)
    _wgrad_check(got, ref, absum)


# ------------------------------------------------------------------ gate backward

def test_gate_backward():
    rng = np.random.default_rng(51)
    T, E, k = 3000, 64, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = OR.topk(lg, k)
    ids[5, 1] = ids[5, 0]                                  # a repeated id sums its slots
    g = (rng.standard_normal((T, k)) * 10.0).astype(np.float32)
    g[9] = 0.0
    say("gate backward")
    got = np64(ops.gate_backward(gpu(g), gpu(w.astype(np.float32)), gpu(ids), E))
    ref = OR.gate_backward(g, w, ids, E)
    bound = 1e-6 * np.max(np.abs(g), axis=1, keepdims=True) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)
    assert np.all(got[9] == 0.0)


# ------------------------------------------------------------------ whole layer

def _train_gpu(wl, x, lg, W13, W2, dy, pow2=False):
    plan = ML.TrainPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, e0=wl.e0, device=DEV, pow2=pow2)
    wts = ML.quantize_weights(W13, W2, transpose=plan.transpose_weights, pow2=pow2)
    plan.forward(x, lg, wts)
    plan.backward(x, dy, wts)
    torch.cuda.synchronize()
    return plan, wts


def _rows(t, rows):
    """Rows of a device tensor, gathered on the device, as numpy (float64 for floats)."""
    sub = t[torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)]
    return np64(sub) if sub.is_floating_point() else npi(sub)


def _cols(t, cols, c0=None, c1=None):
    """t[cols, c0:c1] (rows of a transposed operand, a column range) as numpy;
    a block-transposed operand [rcap/128, cols, 128] is read as [cols, rcap]."""
    idx = torch.as_tensor(np.asarray(cols, dtype=np.int64), device=t.device)
    if t.dim() == 3:
        sub = t[:, idx].permute(1, 0, 2).reshape(len(idx), -1)[:, c0:c1]
    else:
        sub = t[idx][:, c0:c1]
    return np64(sub) if sub.is_floating_point() else npi(sub)


def _sub(t, rows, cols):
    """t[rows][:, cols], both gathered on the device, as float64 numpy."""
    dv = t.device
    return np64(t[:, torch.as_tensor(np.asarray(cols, dtype=np.int64), device=dv)]
                [torch.as_tensor(np.asarray(rows, dtype=np.int64), device=dv)])


def _remap(pr):
    """pair_row restricted to the rows it names: (rows, pair_row over 0..len(rows)-1)."""
    rows = np.unique(pr[pr >= 0])
    out = np.where(pr >= 0, np.searchsorted(rows, np.maximum(pr, 0)), -1)
    return rows, out


def _check_stages(plan, wts, x, dy, wl, rows_of=None, experts=None, feat_of=None, pow2=False):
    """Stage-by-stage parity on the GPU's own upstream operands.

    rows_of(seg) picks the checked rows of an expert's segment (all by default);
    experts restricts the experts; feat_of(m) picks the checked feature rows of
    the transposed operands and weight gradients (all by default)."""
    k, f, d, L = wl.k, wl.f, wl.d, wl.L
    c, o = npi(plan.counts), npi(plan.offsets)
    n = int(o[-1])
    rp = npi(plan.row_pair)[:n]
    real = rp >= 0
    w = np64(plan.w)
    experts = range(L) if experts is None else experts
    rows_of = (lambda seg: seg) if rows_of is None else rows_of
    feat_of = (lambda m: np.arange(m)) if feat_of is None else feat_of
    # inspection rerun of the SwiGLU backward on the same inputs: same bytes
    ins = ops.swiglu_backward(plan.dH, plan.gu, plan.row_pair, plan.offsets, L, plan.rcap, inspect=True, pow2=pow2)
    realrows = np.flatnonzero(real)
    assert torch.equal(ins["dgu_q"][:n][torch.as_tensor(realrows, device=DEV)],
                       plan.sb["dgu_q"][:n][torch.as_tensor(realrows, device=DEV)])
    assert torch.equal(ins["dgu_qT"][:n // 128], plan.sb["dgu_qT"][:n // 128])
    assert torch.equal(ins["h_qT"][:n // 128], plan.sb["h_qT"][:n // 128])
    for e in experts:
        if c[e] == 0:
            continue
        rows = rows_of(np.arange(o[e], o[e] + c[e]))
        t, j = rp[rows] // k, rp[rows] % k
        dys = _rows(dy, t)
        # combine backward: dY = fp32(w * dy), 1x128
        dyq, dyq_s = _rows(plan.dyq, rows), _rows(plan.dyq_s.t(), rows)
        rq, rs = OQ.quant_1x128(of32(w[t, j][:, None] * dys), pow2=pow2)
        assert np.array_equal(dyq, rq) and np.array_equal(dyq_s, rs)
        # dgrad through W2 (transposed copy [f, d]), fp32 accumulators
        # the dgrad products' weights: the forward codes and scales transposed
        w2T, w2sT = npi(wts["w2q"][e]).T, npi(wts["w2s"][e]).T
        ref_dH = OG.blockscaled_matmul(dyq, dyq_s, w2T, OG.expand_weight_scales(w2sT))
        dH = _rows(plan.dH, rows)
        assert rel_fro(dH, ref_dH) <= ACC_TOL
        # SwiGLU backward on the GPU's dH and saved bf16 G, U
        gu = _rows(plan.gu, rows)
        ref_dgu, ref_h = _swiglu_ref(dH, gu[:, :f], gu[:, f:])
        dgu32 = _rows(ins["dgu"], rows)
        assert _tile_close(dgu32, ref_dgu) and _tile_close(_rows(ins["h"], rows), ref_h)
        dgu_q, dgu_s = _rows(plan.sb["dgu_q"], rows), _rows(plan.sb["dgu_s"].t(), rows)
        q1, s1 = OQ.quant_1x128(dgu32, pow2=pow2)
        assert np.array_equal(dgu_q, q1) and np.array_equal(dgu_s, s1)
        # dgrad through W13 (transposed copy [d, 2f]), bf16
        ref_dX = OG.blockscaled_matmul(dgu_q, dgu_s, npi(wts["w13q"][e]).T,
                                       OG.expand_weight_scales(npi(wts["w13s"][e]).T))
        assert rel_fro(_rows(plan.dX, rows), obf16(ref_dX)) <= TOL
    # unpermute-sum of dX, the gate gradient and d_logits on sampled tokens
    toks = np.arange(0, wl.T, max(1, wl.T // 512))
    pr = npi(plan.pair_row)[toks]
    used, prl = _remap(pr)
    assert rel_fro(_rows(plan.dx, toks), OD.combine(_rows(plan.dX, used), prl, None)) <= TOL
    loc = prl >= 0
    Yu = _rows(plan.Y, used)
    prod = _rows(dy, toks)[np.nonzero(loc)[0]] * Yu[prl[loc]]
    dg = _rows(plan.d_gate, toks)
    assert np.all(np.abs(dg[loc] - np.sum(prod, axis=1)) <= 1e-6 * np.sum(np.abs(prod), axis=1) + 1e-30)
    assert np.all(dg[~loc] == 0.0)
    dl = OR.gate_backward(dg, w[toks], npi(plan.ids)[toks], wl.E)
    gmax = np.max(np.abs(dg), axis=1, keepdims=True)
    assert np.all(np.abs(_rows(plan.d_logits, toks) - dl) <= 1e-6 * gmax + 1e-30)
    # 128x1 transposed operands of the wgrad GEMMs, on sampled feature rows
    md, mf, m2f = feat_of(d), feat_of(f), feat_of(2 * f)
    rr = realrows
    Xp = np.zeros((n, len(md)))
    Xp[rr] = _sub(x, rp[rr] // k, md)
    qx, sx = OQ.quant_128x1_t(Xp, real, pow2=pow2)
    assert np.array_equal(_cols(plan.xqT, md, 0, n), qx)
    assert np.array_equal(_cols(plan.xqT_s.t(), md, 0, n // 128), sx)
    dYp = np.zeros((n, len(md)))
    dYp[rr] = of32(w[rp[rr] // k, rp[rr] % k][:, None] * _sub(dy, rp[rr] // k, md))
    qy, sy = OQ.quant_128x1_t(dYp, real, pow2=pow2)
    assert np.array_equal(_cols(plan.dyqT, md, 0, n), qy)
    assert np.array_equal(_cols(plan.dyqT_s.t(), md, 0, n // 128), sy)
    h32 = np.zeros((n, len(mf)))
    h32[rr] = _sub(ins["h"], rr, mf)
    qh, sh = OQ.quant_128x1_t(h32, real, pow2=pow2)
    assert np.array_equal(_cols(plan.sb["h_qT"], mf, 0, n), qh)
    assert np.array_equal(_cols(plan.sb["h_sT"].t(), mf, 0, n // 128), sh)
    g32 = np.zeros((n, len(m2f)))
    g32[rr] = _sub(ins["dgu"], rr, m2f)
    qg, sg = OQ.quant_128x1_t(g32, real, pow2=pow2)
    assert np.array_equal(_cols(plan.sb["dgu_qT"], m2f, 0, n), qg)
    assert np.array_equal(_cols(plan.sb["dgu_sT"].t(), m2f, 0, n // 128), sg)
    # wgrad products, per expert, over the expert's padded segment
    for e in experts:
        lo, hi = int(o[e]), int(o[e + 1])
        seg_c, seg_o = np.array([c[e]]), np.array([0, hi - lo])
        b0, b1 = lo // 128, hi // 128
        def op(qt, st, feats):  # st token-block-major
            return _cols(qt, feats, lo, hi), _cols(st.t(), feats, b0, b1)
        a2, as2 = op(plan.dyqT, plan.dyqT_s, md)
        b2, bs2 = op(plan.sb["h_qT"], plan.sb["h_sT"], np.arange(f))
        ref2 = OG.grouped_wgrad(a2, as2, b2, bs2, seg_c, seg_o)
        abs2 = OG.grouped_wgrad(_abs_codes(a2), as2, _abs_codes(b2), bs2, seg_c, seg_o)
        a13, as13 = op(plan.sb["dgu_qT"], plan.sb["dgu_sT"], m2f)
        b13, bs13 = op(plan.xqT, plan.xqT_s, np.arange(d))
        ref13 = OG.grouped_wgrad(a13, as13, b13, bs13, seg_c, seg_o)
        abs13 = OG.grouped_wgrad(_abs_codes(a13), as13, _abs_codes(b13), bs13, seg_c, seg_o)
        _wgrad_check(_rows(plan.dW2[e], md)[None], ref2, abs2)
        _wgrad_check(_rows(plan.dW13[e], m2f)[None], ref13, abs13)


@pytest.mark.parametrize("pow2", [False, True])
def test_layer_tiny_train(pow2):
    wl = synth.WORKLOADS["tiny"]
    lg = synth.logits(wl)
    x = synth.x(wl)
    dy = synth.dy(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    say(f"tiny layer forward + backward T=128 d=128 f=256 E=8 k=2 pow2={pow2}")
    plan, wts = _train_gpu(wl, x.to(DEV), gpu(lg), W13.to(DEV), W2.to(DEV), dy.to(DEV), pow2=pow2)
    wq = OL.quantize_weights(np64(W13), np64(W2), pow2=pow2)
    assert np.array_equal(npi(wts["w13qT"]), np.swapaxes(wq[0][0], 1, 2))
    assert np.array_equal(npi(wts["w2qT"]), np.swapaxes(wq[1][0], 1, 2))
    _check_stages(plan, wts, x.to(DEV), dy.to(DEV), wl, pow2=pow2)
    # end to end against the oracle's own chain: the two chains take their FP8
    # decisions on values that differ by fp32 rounding, so an occasional code
    # lands one step apart; 1e-2 bounds that effect at this size.
    ids, w = OR.topk(lg, wl.k)
    fw = OL.forward(np64(x), ids, w, 0, wl.L, wq, pow2=pow2)
    bw = OL.backward(fw, np64(dy), ids, w, wl.E, wq, pow2=pow2)
    for name, got, ref in (("dx", plan.dx, bw["dx"]), ("dW2", plan.dW2, bw["dW2"]),
                           ("dW13", plan.dW13, bw["dW13"]), ("d_logits", plan.d_logits, bw["d_logits"])):
        err = rel_fro(np64(got), ref)
        say(f"tiny chain {name}: rel err {err:.2e}")
        assert err <= 1e-2, name


@pytest.mark.parametrize("pow2", [False, True])
def test_layer_train_full_size_sampled(pow2):
    """T=16384, d=7168, f=2048, 32 of 256 experts, top-8, forward + backward,
    launched as the benchmark launches it; stages checked on sampled rows."""
    wl = synth.WORKLOADS["train"]
    say("train: generating inputs")
    lg = synth.logits(wl)
    x = synth.x(wl)
    dy = synth.dy(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    say(f"train: GPU forward + backward pow2={pow2}")
    plan, wts = _train_gpu(wl, x.to(DEV), gpu(lg), W13.to(DEV), W2.to(DEV), dy.to(DEV), pow2=pow2)
    ids, w = OR.topk(lg, wl.k)
    assert np.array_equal(npi(plan.ids), ids)
    c, o, rp, pr = OD.permute_index(ids, wl.e0, wl.L)
    assert np.array_equal(npi(plan.counts), c) and np.array_equal(npi(plan.offsets), o)
    assert np.array_equal(npi(plan.pair_row), pr)
    say("train: indices bit-exact; forward stages (GEMM1 saving G/U, GEMM2, combine) on sampled rows")
    h32 = LC.gemm1_h32(plan.xq, plan.xq_s, wts["w13q"], wts["w13s"], plan.counts, plan.offsets, pow2=pow2,
                       thin_ws=plan.thin_ws)
    LC.check_layer_forward(wl, x, W13, W2, plan, h32, (0, 13, 31), wts=wts, pow2=pow2, save_gu=True, n_rows=16,
                           tok_stride=131, tag="train")
    del h32, W13, W2
    say("train: backward stages on sampled rows")
    _check_stages(plan, wts, x.to(DEV), dy.to(DEV), wl,
                  rows_of=lambda seg: seg[:: max(1, len(seg) // 16)], experts=(0, 13, 31),
                  feat_of=lambda m: np.arange(0, m, m // 32), pow2=pow2)
    say("train sampled parity ok")


# ------------------------------------------------------------------ determinism

def _plan_tensors(plan):
    """Every device buffer a training step writes (the status word and the
    permute workspace aside)."""
    out = {n: t for n, t in vars(plan).items() if isinstance(t, torch.Tensor) and n not in ("status", "ws")}
    out.update({f"sb.{n}": t for n, t in plan.sb.items()})
    return out


def _poison(tensors):
    for t in tensors.values():
        if t.dtype.is_floating_point:
            t.fill_(-7.0e30)
        elif t.dtype == torch.uint8:
            t.fill_(0xA5)
        else:
            t.fill_(-123456789)


def test_train_step_run_twice_bitwise():
    """The full training step (T=16384, d=7168, f=2048, 32 of 256 experts,
    top-8) twice on the same inputs, every buffer overwritten with the same
    poison before each run: every output, intermediate and index buffer is
    bitwise equal (the path has no order-dependent atomics), so no element is
    left unwritten in one run and written in the other."""
    wl = synth.WORKLOADS["train"]
    say("run twice: inputs")
    x = synth.x(wl).to(DEV)
    lg = gpu(synth.logits(wl))
    dy = synth.dy(wl).to(DEV)
    plan = ML.TrainPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, e0=wl.e0, device=DEV)
    wts = ML.quantize_weights(synth.weights(wl, "w13").to(DEV), synth.weights(wl, "w2").to(DEV),
                              transpose=plan.transpose_weights)
    bufs = _plan_tensors(plan)
    runs = []
    for i in range(2):
        _poison(bufs)
        plan.status.zero_()
        plan.forward(x, lg, wts)
        plan.backward(x, dy, wts)
        torch.cuda.synchronize()
        say(f"run twice: run {i} done")
        runs.append({n: t.clone() for n, t in bufs.items()} if i == 0 else bufs)
    assert int(plan.status.item()) == 0
    differ = [n for n in bufs if not torch.equal(runs[0][n], runs[1][n])]
    assert not differ, f"buffers differ between two runs: {differ}"


# ------------------------------------------------------------------ end to end against the oracle's own chain

_E4M3_GRID = None


def _grid_index(codes):
    """Position of each e4m3 code's value in the sorted grid of finite e4m3
    values (both zeros share one position)."""
    global _E4M3_GRID
    from oracle.numerics import e4m3_decode
    if _E4M3_GRID is None:
        allv = e4m3_decode(np.arange(256, dtype=np.uint8))
        _E4M3_GRID = np.unique(allv[np.isfinite(allv)])
    return np.searchsorted(_E4M3_GRID, e4m3_decode(codes))


def _flips(name, q_gpu, s_gpu, q_ref, s_ref, v_gpu, v_ref, tile_axis, exempt=None):
    """Compare two FP8 quantisations of nearly equal values (the GPU chain's
    fp32 values and the oracle chain's): codes and scales, tiles of 128 along
    tile_axis.  The two underlying values must differ by no more than 1e-4 of
    the tile's largest magnitude, and every differing code must be the e4m3
    neighbour of the other (one rounding decision on the other side of a
    midpoint) or lie next to zero: the flips come from the fp32-vs-fp64
    values, not from the quantiser (whose codes on the GPU's own values are
    checked bit-exact stage by stage).  ``exempt`` marks elements computed from a
    bf16 value that itself rounded one bf16 step apart in the two chains (the
    saved G and U): they are only counted.  Returns
    (differing codes, codes, tiles whose scale differs)."""
    q_gpu, q_ref = np.asarray(q_gpu), np.asarray(q_ref)
    v_gpu, v_ref = np.asarray(v_gpu, np.float64), np.asarray(v_ref, np.float64)
    s_gpu, s_ref = np.asarray(s_gpu, np.float64), np.asarray(s_ref, np.float64)
    exempt = np.zeros(np.shape(q_gpu), bool) if exempt is None else np.asarray(exempt)
    if tile_axis == 0:
        q_gpu, q_ref, v_gpu, v_ref, s_gpu, s_ref = q_gpu.T, q_ref.T, v_gpu.T, v_ref.T, s_gpu.T, s_ref.T
        exempt = exempt.T
    rows, cols = q_gpu.shape
    amax = np.repeat(np.max(np.abs(v_ref).reshape(rows, cols // 128, 128), axis=2), 128, axis=1)
    diff = q_gpu != q_ref
    own = diff & ~exempt
    close = (np.abs(v_gpu - v_ref) <= 1e-4 * amax) | exempt
    assert np.all(close), f"{name}: fp32 values differ by more than 1e-4 of their tile max"
    # every differing code is the e4m3 neighbour of the other, or both scaled
    # values lie within two subnormal steps of zero (the sign of a value near
    # zero differs between the chains: -2^-9 and +2^-9 are two grid positions)
    sg = np.repeat(s_gpu, 128, axis=1)
    sr = np.repeat(s_ref, 128, axis=1)
    near0 = (np.abs(v_gpu / sg) < 2.0 ** -8) & (np.abs(v_ref / sr) < 2.0 ** -8)
    nd, nx = int(np.count_nonzero(own)), int(np.count_nonzero(diff & exempt))
    if nd:
        step = np.abs(_grid_index(q_gpu[own]) - _grid_index(q_ref[own]))
        ok = (step == 1) | near0[own]
        assert np.all(ok), (f"{name}: codes {q_gpu[own][~ok][:4]} vs {q_ref[own][~ok][:4]} for values "
                            f"{v_gpu[own][~ok][:4]} vs {v_ref[own][~ok][:4]}")
    ns = int(np.count_nonzero(s_gpu != s_ref))
    say(f"  {name}: {nd} of {diff.size} codes one e4m3 step apart (or both next to zero), {nx} more downstream "
        f"of a saved G/U bf16 flip; {ns} of {s_gpu.size} tile scales differ")
    return nd, diff.size, ns


def _count_flips(name, q_gpu, q_ref):
    """Codes that differ between the GPU chain and the oracle chain at a
    rounding point downstream of earlier differences (counted, not bounded)."""
    nd = int(np.count_nonzero(np.asarray(q_gpu) != np.asarray(q_ref)))
    say(f"  {name}: {nd} of {np.size(q_gpu)} codes differ")
    return nd


@pytest.mark.parametrize("pow2", [False, True])
def test_tiny_train_end_to_end_explained(pow2):
    """Why the GPU chain differs from the oracle's own FP8 chain end to end
    (a few 1e-3 on dx and dW13) while every stage meets 2e-3 on the GPU's own
    operands.  The two chains round at the same points (gates to fp32, h and
    every backward operand to e4m3, G/U and Y to bf16) but from values that
    differ in their last bits (fp32 accumulation and expf on the GPU, fp64 in
    the oracle), so a few rounding decisions fall on the other side of a
    midpoint, and each such difference propagates:
      1. where both chains start from identical FP8 operands (GEMM1 over the
         same Xq and W13 codes) the fp32 values agree to 1e-4 of the tile or
         row maximum, and every code or bf16 value that differs is one step
         from the oracle's, at a midpoint between the two values;
      2. the gates agree to 1e-6, and the downstream points (dY, dGU, H) are
         counted: their codes differ where upstream differences reach them;
      3. the oracle run on the GPU's own rounded values at every rounding point
         reproduces every GPU output (y, dx, dW2, dW13, d_logits) within 2e-3.
    So the end-to-end gap is the propagation of those few rounding decisions,
    not kernel error; the 1e-2 end-to-end bound below rests on this."""
    wl = synth.WORKLOADS["tiny"]
    lg = synth.logits(wl)
    x = synth.x(wl)
    dy = synth.dy(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    say(f"tiny train end to end, pow2={pow2}")
    plan, wts = _train_gpu(wl, x.to(DEV), gpu(lg), W13.to(DEV), W2.to(DEV), dy.to(DEV), pow2=pow2)
    ids, w = OR.topk(lg, wl.k)
    wq = OL.quantize_weights(np64(W13), np64(W2), pow2=pow2)
    fw = OL.forward(np64(x), ids, w, 0, wl.L, wq, pow2=pow2)
    bw = OL.backward(fw, np64(dy), ids, w, wl.E, wq, pow2=pow2)
    n = int(npi(plan.offsets)[-1])
    rp = npi(plan.row_pair)[:n]
    real = rp >= 0
    rr = np.flatnonzero(real)
    act = lambda v: OQ.quant_1x128(v, pow2=pow2)
    act_t = lambda v: OQ.quant_128x1_t(v, real, pow2=pow2)
    say("1. rounding points fed by identical FP8 operands")
    assert np.array_equal(npi(plan.xq)[rr], fw["Xa"][0][rr])
    h32 = np64(LC.gemm1_h32(plan.xq, plan.xq_s, wts["w13q"], wts["w13s"], plan.counts, plan.offsets, pow2=pow2,
                            thin_ws=plan.thin_ws))
    hq_o, hs_o = fw["ha"]
    _flips("h 1x128", npi(plan.hq)[rr], npi(plan.hq_s).T[rr], hq_o[rr], hs_o[rr], h32[rr], fw["h"][rr], 1)
    # the saved bf16 G, U: the GPU rounds its own fp32 accumulators (the
    # STORE_F32 dump of the same GEMM), which agree with the oracle's fp64 G, U
    # to 1e-4 of the row maximum; a saved value differs from the oracle's only
    # by the one bf16 step of a midpoint between the two values
    gu32 = np64(ops.grouped_gemm(plan.xq, plan.xq_s, wts["w13q"], wts["w13s"], plan.counts, plan.offsets,
                                 ops.EPI_STORE_F32, pow2=pow2))[:n]
    GU_o = np.concatenate([fw["G"], fw["U"]], axis=1)[:n]
    assert np.array_equal(np64(plan.gu)[rr], obf16(gu32[rr]))
    rmax = np.max(np.abs(GU_o[rr]), axis=1, keepdims=True)
    assert np.all(np.abs(gu32[rr] - GU_o[rr]) <= 1e-4 * rmax)
    gu_ref = obf16(GU_o)
    gu_flip = (np64(plan.gu)[:n] != gu_ref) & real[:, None]
    lo, hi = np.minimum(gu32, GU_o)[gu_flip], np.maximum(gu32, GU_o)[gu_flip]
    mid = (np64(plan.gu)[:n][gu_flip] + gu_ref[gu_flip]) / 2          # the bf16 midpoint between the two
    assert np.all((lo <= mid) & (mid <= hi))
    say(f"  saved G/U bf16: {int(np.count_nonzero(gu_flip))} of {gu_flip[rr].size} values one bf16 step apart, "
        "each at a midpoint between the GPU's fp32 value and the oracle's")
    say("2. gates and downstream rounding points")
    gw = np64(plan.w)
    assert np.max(np.abs(gw - w)) <= 1e-6
    say(f"  gates: {int(np.count_nonzero(gw != w))} of {w.size} fp32 values differ (by at most 1e-6)")
    _count_flips("dY 1x128", npi(plan.dyq)[rr], act(bw["dYp"])[0][rr])
    _count_flips("dGU 1x128", npi(plan.sb["dgu_q"])[rr], act(bw["dGU"])[0][rr])
    _count_flips("dGU 128x1", npi(ops.untile_t(plan.sb["dgu_qT"]))[:, :n], act_t(bw["dGU"])[0])
    _count_flips("H 128x1", npi(ops.untile_t(plan.sb["h_qT"]))[:, :n],
                 act_t(np.where(real[:, None], bw["Hr"], 0.0))[0])
    say("3. the oracle on the GPU's rounded values reproduces every GPU output within 2e-3")
    c, o = npi(plan.counts), npi(plan.offsets)
    pr = npi(plan.pair_row)
    Y_o = obf16(OG.grouped_forward(npi(plan.hq), npi(plan.hq_s).T, c, o, wq[1][0], wq[1][1]))
    y_o = OD.combine(Y_o, pr, gw)
    dX_o = obf16(OG.grouped_dgrad(npi(plan.sb["dgu_q"]), npi(plan.sb["dgu_s"]).T, c, o, wq[0][0], wq[0][1]))
    dx_o = OD.combine(dX_o, pr, None)
    gq = lambda qT, sT: (npi(ops.untile_t(qT))[:, :n], npi(sT)[:n // 128].T)
    dW2_o = obf16(OG.grouped_wgrad(*gq(plan.dyqT, plan.dyqT_s), *gq(plan.sb["h_qT"], plan.sb["h_sT"]), c, o))
    dW13_o = obf16(OG.grouped_wgrad(*gq(plan.sb["dgu_qT"], plan.sb["dgu_sT"]), *gq(plan.xqT, plan.xqT_s), c, o))
    Yg = np64(plan.Y)
    d_gate_o = np.zeros((wl.T, wl.k))
    loc = pr >= 0
    d_gate_o[loc] = np.sum(np64(dy)[np.nonzero(loc)[0]] * Yg[pr[loc]], axis=1)
    dl_o = OR.gate_backward(d_gate_o, gw, ids, wl.E)
    for name, got, ref_codes, ref_own in (("y", plan.y, y_o, fw["y"]), ("dx", plan.dx, dx_o, bw["dx"]),
                                          ("dW2", plan.dW2, dW2_o, bw["dW2"]),
                                          ("dW13", plan.dW13, dW13_o, bw["dW13"]),
                                          ("d_logits", plan.d_logits, dl_o, bw["d_logits"])):
        g = np64(got)
        e_codes = rel_fro(g, ref_codes)
        e_own = rel_fro(g, ref_own)
        e_between = rel_fro(ref_codes, ref_own)
        say(f"  {name}: GPU vs oracle on the GPU's rounded values {e_codes:.2e}; GPU vs oracle's own chain "
            f"{e_own:.2e}; the two oracle runs {e_between:.2e}")
        assert e_codes <= TOL, name
        assert e_own <= 1e-2, name


def test_train_step_graph_replay():
    """The training step as the benchmark replays it: weights re-quantised,
    forward and backward captured into one HIP graph per input set.  Each
    replay, with eager steps and synchronisations in between and every buffer
    poisoned first, writes bit for bit what the eager step writes on the same
    inputs."""
    wl = synth.WORKLOADS["train"]
    say("train graph: inputs")
    xs = [synth.x(wl, t0=i * wl.T).to(DEV) for i in range(2)]
    lgs = [gpu(synth.logits(wl, t0=i * wl.T)) for i in range(2)]
    dys = [synth.dy(wl, t0=i * wl.T).to(DEV) for i in range(2)]
    W13 = synth.weights(wl, "w13").to(DEV)
    W2 = synth.weights(wl, "w2").to(DEV)
    plan = ML.TrainPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, e0=wl.e0, device=DEV)
    wts = ML.weight_buffers(wl.L, wl.d, wl.f, DEV, transpose=plan.transpose_weights)

    def step(i):
        ML.quantize_weights(W13, W2, transpose=plan.transpose_weights, out=wts)
        plan.forward(xs[i], lgs[i], wts)
        plan.backward(xs[i], dys[i], wts)

    say("train graph: capture")
    graphs = [ML.capture_graph(lambda i=i: step(i)) for i in range(2)]
    bufs = _plan_tensors(plan)
    bufs.update({f"wts.{n}": t for n, t in wts.items()})
    for it in (1, 0, 1, 0):
        _poison(bufs)
        step(it)
        torch.cuda.synchronize()
        ref = {n: t.clone() for n, t in bufs.items()}
        _poison(bufs)
        graphs[it].replay()
        torch.cuda.synchronize()
        say(f"train graph: replay with input set {it}")
        differ = [n for n in bufs if not torch.equal(bufs[n], ref[n])]
        assert not differ, f"graph replay differs from the eager step in {differ}"
        del ref
    assert int(plan.status.item()) == 0
