"""Full-size parity checks shared by the GPU layer tests (not collected by pytest).

Each check compares a stage of the GPU path with the oracle on sampled rows,
with the oracle run over the very FP8 operands the GPU produced upstream:

  * GEMM1 + SwiGLU: the GPU's fp32 h (the SWIGLU_F32 epilogue dump of the same
    GEMM on the same operands) within ACC_TOL of the oracle's fp64 block
    accumulation, and the fused 1x128 codes and scales of the production
    epilogue bit-exact against the oracle's quantiser applied to that h;
  * GEMM2: bf16 Y within TOL relative Frobenius;
  * combine: every element within one bf16 ulp of the exact weighted sum plus
    the bound of an fp32 accumulation of k products."""

import numpy as np
import torch

from oracle import blockfp8 as OQ
from oracle import dispatch as OD
from oracle import gemm as OG
from oracle import layer as OL
from oracle import mxfp4 as MX
from oracle import routing as OR
from oracle.numerics import bf16 as obf16, f32 as of32
from moe_expert_layer_r3_amd import ops, synth
from gpu_util import DEV, gpu, np64, npi, rel_fro, say

TOL = 2e-3
ACC_TOL = 1e-4


def sample_rows(o, c, e, n=24):
    """Rows of expert e's segment to check: a stride over the segment, the rows
    on both sides of every 128- and 256-row tile boundary inside it, and its
    last four rows (where a partly filled 16-row MFMA subtile is stored)."""
    lo, cnt = int(o[e]), int(c[e])
    if cnt == 0:
        return np.zeros(0, dtype=np.int64)
    rel = set(range(0, cnt, max(1, cnt // n)))
    rel.update(range(max(0, cnt - 4), cnt))
    for b in range(128, cnt, 128):
        rel.update((b - 1, b))
    return lo + np.array(sorted(rel), dtype=np.int64)


def rows_of(t, rows):
    """t[rows] gathered on the device, as numpy (float64 for float tensors)."""
    sub = t[torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)]
    return np64(sub) if sub.is_floating_point() else npi(sub)


def gemm1_h32(xq, xq_s, w13q, w13s, counts, offsets, pow2=False, mxfp4=False, thin_ws=None):
    """The GPU's fp32 h = silu(G) * U before quantisation: the same grouped GEMM
    with the SWIGLU_F32 inspection epilogue (and, with the plan's thin_ws, the
    same K-split path for thin last m-tiles as the plan's GEMM1)."""
    return ops.grouped_gemm(xq, xq_s, w13q, w13s, counts, offsets, ops.EPI_SWIGLU_F32, pow2=pow2, mxfp4=mxfp4,
                            thin_ws=thin_ws)


def expert_weights_checked(e, W13e, W2e, wts=None, pow2=False, mxfp4=False):
    """One expert's oracle-quantised weights, as the operands of ``matmul``:
    ((codes13, scales13), (codes2, scales2)), 128x128 FP8 with the block scales
    expanded to one per row, or MXFP4 codes and E8M0 scale codes.  With ``wts``
    (the GPU's quantised weights) the GPU's codes and scales of expert e are
    first checked bit-exact against them."""
    if mxfp4:
        wq = MX.quant_mx(np64(W13e)), MX.quant_mx(np64(W2e))
        if wts is not None:
            for (qc, sc), q, s in ((wq[0], "w13q", "w13s"), (wq[1], "w2q", "w2s")):
                assert np.array_equal(MX.unpack(ops.mx_codes_rows(wts[q][e:e + 1])[0]), qc), f"expert {e} {q}"
                assert np.array_equal(ops.mx_scales_rows(wts[s][e:e + 1])[0], sc), f"expert {e} {s}"
        return wq
    out = []
    for W, q, s in ((W13e, "w13q", "w13s"), (W2e, "w2q", "w2s")):
        rq, rs = OQ.quant_128x128(np64(W)[None], pow2=pow2)
        if wts is not None:
            assert np.array_equal(npi(wts[q][e]), rq[0]), f"expert {e} {q}"
            assert np.array_equal(npi(wts[s][e]).astype(np.float64), rs[0]), f"expert {e} {s}"
        out.append((rq[0], OG.expand_weight_scales(rs[0])))
    return tuple(out)


def matmul(qa, sa, wq, mxfp4=False):
    return MX.matmul(qa, sa, *wq) if mxfp4 else OG.blockscaled_matmul(qa, sa, *wq)


def check_expert_forward(e, rows, f, xq, xq_s, h32, hq, hq_s, Y, wq, pow2=False, mxfp4=False, gu=None,
                         x_rows=None):
    """GEMM1 (fp32 h, fused codes, saved G/U) and GEMM2 on the given rows of
    expert e, over the GPU's own Xq and hq; wq from expert_weights_checked.
    x_rows: the bf16 token rows those rows hold, to check Xq bit-exact."""
    p2 = pow2 or mxfp4
    xq_r = rows_of(xq, rows)
    xs_r = rows_of(xq_s.t(), rows)
    if x_rows is not None:
        rq, rs = OQ.quant_1x128(x_rows, pow2=p2)
        assert np.array_equal(xq_r, rq) and np.array_equal(xs_r, rs), f"expert {e}: Xq bytes differ"
    GU = matmul(xq_r, xs_r, wq[0], mxfp4)
    G, U = of32(GU[:, :f]), of32(GU[:, f:])
    h_ref = OL.silu(G) * U
    h_gpu = rows_of(h32, rows)
    eh = rel_fro(h_gpu, h_ref)
    assert eh <= ACC_TOL, f"expert {e}: fp32 h rel err {eh:.3e} > {ACC_TOL}"
    qref, sref = OQ.quant_1x128(h_gpu, pow2=p2)
    hq_r = rows_of(hq, rows)
    hs_r = rows_of(hq_s.t(), rows)
    bad = np.count_nonzero(hq_r != qref)
    assert bad == 0, f"expert {e}: {bad} fused h codes differ from the oracle's quantiser"
    assert np.array_equal(hs_r, sref), f"expert {e}: fused h scales differ"
    if gu is not None:
        eg = rel_fro(rows_of(gu, rows), obf16(GU))
        assert eg <= TOL, f"expert {e}: saved G/U rel err {eg:.3e}"
    Yref = obf16(matmul(hq_r, hs_r, wq[1], mxfp4))
    ey = rel_fro(rows_of(Y, rows), Yref)
    assert ey <= TOL, f"expert {e}: Y rel err {ey:.3e}"
    return eh, ey


def check_combine_elementwise(y_gpu, Y_rows, pair_row, w):
    """y_gpu [n, d] for n tokens whose slots pair_row [n, k] index Y_rows (rows of
    the GPU's Y, -1 = non-local), gates w [n, k] (None = weights 1).

    The library sums fp32 products in slot order and rounds once to bf16, so
    each element lies within one bf16 ulp of the exact sum s plus the fp32
    accumulation bound 2k * 2^-24 * sum |w Y|.  Returns the number of elements
    that differ from bf16(s) (a rounding decision taken on the other side of a
    bf16 midpoint)."""
    n, k = pair_row.shape
    d = Y_rows.shape[1]
    s = np.zeros((n, d))
    a = np.zeros((n, d))
    for j in range(k):
        r = pair_row[:, j]
        m = r >= 0
        wj = 1.0 if w is None else np.asarray(w, np.float64)[m, j][:, None]
        term = wj * Y_rows[r[m]]
        s[m] += term
        a[m] += np.abs(term)
    got = np.asarray(y_gpu, np.float64)
    mag = np.maximum(np.abs(got), np.abs(s))
    ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.maximum(mag, 1e-300))) - 7), 0.0)
    bound = ulp + 2 * k * 2.0 ** -24 * a
    err = np.abs(got - s)
    if not np.all(err <= bound):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"combine element {i}: got {got[i]!r}, exact sum {s[i]!r}, bound {bound[i]!r}")
    none = np.all(pair_row < 0, axis=1)
    assert np.all(got[none] == 0.0)
    return int(np.count_nonzero(got != obf16(s)))


def check_layer_forward(wl, x, W13, W2, plan, h32, experts, wts=None, pow2=False, mxfp4=False, save_gu=False,
                        n_rows=24, tok_stride=97, tag=""):
    """Sampled GEMM1/GEMM2 rows of the given experts and the combine on every
    tok_stride-th token, against the oracle over the GPU's own operands.
    plan: the GPU forward's buffers (xq, xq_s, hq, hq_s, Y, y, counts, offsets,
    row_pair, pair_row, w, gu), x the host bf16 input, W13 / W2 the host bf16
    weights, wts the GPU's quantised weights (checked bit-exact when given)."""
    c, o = npi(plan.counts), npi(plan.offsets)
    rp = npi(plan.row_pair)[:int(o[-1])]
    for e in experts:
        rows = sample_rows(o, c, e, n_rows)
        if len(rows) == 0:
            continue
        wq = expert_weights_checked(e, W13[e], W2[e], wts, pow2=pow2, mxfp4=mxfp4)
        x_rows = np64(x[torch.as_tensor(rp[rows] // wl.k)])
        eh, ey = check_expert_forward(e, rows, wl.f, plan.xq, plan.xq_s, h32, plan.hq, plan.hq_s, plan.Y, wq,
                                      pow2=pow2, mxfp4=mxfp4, gu=plan.gu if save_gu else None, x_rows=x_rows)
        say(f"{tag} expert {e} ({c[e]} rows, {len(rows)} checked): h {eh:.2e}, Y {ey:.2e}")
    toks = np.arange(0, wl.T, tok_stride)
    pr = npi(plan.pair_row)[toks]
    used = np.unique(pr[pr >= 0])
    prl = np.where(pr >= 0, np.searchsorted(used, np.maximum(pr, 0)), -1)
    flips = check_combine_elementwise(rows_of(plan.y, toks), rows_of(plan.Y, used), prl, np64(plan.w)[toks])
    say(f"{tag} combine: {len(toks)} tokens per element, {flips} elements one bf16 step from bf16(exact)")


def _plan_forward(wl, pow2=False, mxfp4=False, save_gu=False):
    """The forward through ForwardPlan on the workload's seeded inputs, launched
    as the benchmark launches it; returns the host inputs, weights and plan."""
    from moe_expert_layer_r3_amd.layer import ForwardPlan, quantize_weights
    say(f"{wl.name}: generating inputs")
    lg = synth.logits(wl)
    x = synth.x(wl)
    W13 = synth.weights(wl, "w13")
    W2 = synth.weights(wl, "w2")
    say(f"{wl.name}: GPU forward pow2={pow2} mxfp4={mxfp4}")
    wts = quantize_weights(W13.to(DEV), W2.to(DEV), pow2=pow2, mxfp4=mxfp4)
    plan = ForwardPlan(wl.T, wl.d, wl.f, wl.E, wl.L, wl.k, wl.e0, device=DEV, pow2=pow2, mxfp4=mxfp4,
                       save_gu=save_gu)
    plan.forward(x.to(DEV), gpu(lg), wts)
    torch.cuda.synchronize()
    return lg, x, W13, W2, wts, plan


def full_size_forward_check(wl, experts, pow2=False, mxfp4=False, n_rows=24, tok_stride=97):
    """Routing and permutation indices bit-exact; GEMM1 at full K (fp32 h within
    1e-4, fused h codes bit-exact), GEMM2 within 2e-3 and the combine per element
    on sampled rows of the given experts (None: hottest, median and coldest)."""
    lg, x, W13, W2, wts, plan = _plan_forward(wl, pow2=pow2, mxfp4=mxfp4)
    ids, w = OR.topk(lg, wl.k)
    assert np.array_equal(npi(plan.ids), ids)
    assert np.max(np.abs(np64(plan.w) - w)) <= 1e-6
    c, o, rp, pr = OD.permute_index(ids, wl.e0, wl.L)
    assert np.array_equal(npi(plan.counts), c) and np.array_equal(npi(plan.offsets), o)
    assert np.array_equal(npi(plan.pair_row), pr)
    n = int(o[-1])
    assert np.array_equal(npi(plan.row_pair)[:n], rp)
    say(f"{wl.name}: indices bit-exact; fp32 h dump and sampled rows")
    if experts is None:
        experts = (int(np.argmax(c)), int(np.argsort(c)[len(c) // 2]), int(np.argmin(c)))
    h32 = gemm1_h32(plan.xq, plan.xq_s, wts["w13q"], wts["w13s"], plan.counts, plan.offsets,
                    pow2=pow2 or mxfp4, mxfp4=mxfp4, thin_ws=plan.thin_ws)
    check_layer_forward(wl, x, W13, W2, plan, h32, experts, wts=wts, pow2=pow2, mxfp4=mxfp4,
                        n_rows=n_rows, tok_stride=tok_stride, tag=wl.name)
    say(f"{wl.name} sampled parity ok")
