"""The MoE expert layer on one GPU's share of experts, as a sequence of C-ABI
calls on preallocated device buffers (no allocation per step).

Forward:  route (top-k, or Router Replay of recorded ids) -> permute + gather +
1x128 FP8 quant -> grouped GEMM1 with fused SwiGLU + 1x128 quant -> grouped
GEMM2 -> weighted combine.  Weights are quantised once per weight version
(128x128 tiles) by ``quantize_weights``."""

import torch

from . import ops
from .ops import _call, _p, _stream


def _check(t, shape, dtype, name):
    """Caller tensors must match the plan's sizes: the kernels index them by the
    plan's T, d, E, and a smaller tensor would be read past its end."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def weight_buffers(L, d, f, device="cuda", transpose=False):
    """Preallocated FP8 weight codes and scales for quantize_weights(out=...)."""
    u8, f32 = torch.uint8, torch.float32
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
    out = dict(w13q=e((L, 2 * f, d), u8), w13s=e((L, 2 * f // 128, d // 128), f32),
               w2q=e((L, d, f), u8), w2s=e((L, d // 128, f // 128), f32))
    if transpose:
        out.update(w13qT=e((L, d, 2 * f), u8), w13sT=e((L, d // 128, 2 * f // 128), f32),
                   w2qT=e((L, f, d), u8), w2sT=e((L, f // 128, d // 128), f32))
    return out


def quantize_weights(W13, W2, transpose=False, out=None, pow2=False, mxfp4=False):
    """bf16 W13 [L, 2f, d], W2 [L, d, f] -> dict of FP8 codes and scales (and the
    transposed copies used by the dgrad GEMMs when ``transpose``), 128x128 tiles,
    power-of-two scales when ``pow2``.  ``mxfp4``: MXFP4 weights instead (forward
    GEMMs only): w13q [L, d/128, 2f, 64] packed E2M1, w13s [L, d/128, 2f, 4]
    E8M0 codes (both K-block-major), and alike for W2.
    ``out`` (from weight_buffers) receives the result without allocating."""
    L, f2, d = W13.shape
    # the output buffers are sized from W13: W2 must be its [L, d, f] partner
    _check(W13, (L, f2, d), torch.bfloat16, "W13")
    _check(W2, (L, d, f2 // 2), torch.bfloat16, "W2")
    if mxfp4:
        e = lambda shape: torch.empty(shape, dtype=torch.uint8, device=W13.device)
        f = f2 // 2
        if out is None:
            out = dict(w13q=e((L, d // 128, f2, 64)), w13s=e((L, d // 128, f2, 4)),
                       w2q=e((L, f // 128, d, 64)), w2s=e((L, f // 128, d, 4)))
            if transpose:  # for the dgrad products: blocks along the other axis
                out.update(w13qT=e((L, f2 // 128, d, 64)), w13sT=e((L, f2 // 128, d, 4)),
                           w2qT=e((L, d // 128, f, 64)), w2sT=e((L, d // 128, f, 4)))
        for W, q, s in ((W13, "w13q", "w13s"), (W2, "w2q", "w2s")):
            if W.dtype != torch.bfloat16 or not W.is_contiguous():
                raise ValueError("weights must be contiguous bf16")
            qT, sT = (out[q + "T"], out[s + "T"]) if transpose else (None, None)
            _call("moe_quant_mxfp4", _p(W), W.shape[0], W.shape[1], W.shape[2], W.shape[2], _p(out[q]), _p(out[s]),
                  _p(qT), _p(sT), _stream())
        return out
    if out is None:
        out = weight_buffers(L, d, f2 // 2, W13.device, transpose)
    for W, q, s in ((W13, "w13q", "w13s"), (W2, "w2q", "w2s")):
        if W.dtype != torch.bfloat16 or not W.is_contiguous():
            raise ValueError("weights must be contiguous bf16")
        _, rows, cols = W.shape
        qT, sT = (out[q + "T"], out[s + "T"]) if transpose else (None, None)
        tile = ops.TILE_128x128 | (ops.SCALE_POW2 if pow2 else 0)
        _call("moe_quant_fp8", _p(W), ops.SRC_BF16, L, rows, cols, cols, tile, _p(out[q]), _p(out[s]),
              _p(qT), _p(sT), _stream())
    return out


class ForwardPlan:
    """Device buffers for one forward pass of T tokens.  pow2: power-of-two
    (UE8M0) activation scales, applied by the MFMA; the weights must then come
    from quantize_weights(..., pow2=True).  mxfp4: MXFP4 weights (from
    quantize_weights(..., mxfp4=True)) with power-of-two FP8 activations."""

    def __init__(self, T, d, f, E, L, k, e0=0, device="cuda", save_gu=False, pow2=False, mxfp4=False):
        self.T, self.d, self.f, self.E, self.L, self.k, self.e0 = T, d, f, E, L, k, e0
        self.sflag = ops.SCALE_POW2 if (pow2 or mxfp4) else 0  # activation quantisers
        self.gflag = self.sflag | (ops.WEIGHT_MXFP4 if mxfp4 else 0)  # forward GEMMs
        self.rcap = ops.row_cap(T, k, L)
        dv = device
        i32, f32, u8, b16 = torch.int32, torch.float32, torch.uint8, torch.bfloat16
        R = self.rcap
        self.ids = torch.empty((T, k), dtype=i32, device=dv)
        self.w = torch.empty((T, k), dtype=f32, device=dv)
        self.counts = torch.empty(L, dtype=i32, device=dv)
        self.offsets = torch.empty(L + 1, dtype=i32, device=dv)
        self.row_pair = torch.empty(R, dtype=i32, device=dv)
        self.pair_row = torch.empty((T, k), dtype=i32, device=dv)
        self.ws = torch.empty(ops.permute_workspace(T, k, L), dtype=u8, device=dv)
        self.status = torch.zeros(1, dtype=i32, device=dv)
        self.xq = torch.empty((R, d), dtype=u8, device=dv)
        self.xq_s = torch.empty((d // 128, R), dtype=f32, device=dv)  # activation scales: K-block-major
        self.hq = torch.empty((R, f), dtype=u8, device=dv)
        self.hq_s = torch.empty((f // 128, R), dtype=f32, device=dv)
        self.gu = torch.empty((R, 2 * f), dtype=b16, device=dv) if save_gu else None
        # workspace of GEMM1's K-split thin m-tiles (FP8 weights)
        self.thin_ws = None if mxfp4 else torch.empty(ops.thin_workspace(L, 2 * f, d), dtype=u8, device=dv)
        self.Y = torch.empty((R, d), dtype=b16, device=dv)
        self.y = torch.empty((T, d), dtype=b16, device=dv)

    # each stage is one C-ABI call on the current stream
    def route(self, logits):
        _check(logits, (self.T, self.E), torch.float32, "logits")
        _call("moe_route_topk", _p(logits), self.T, self.E, self.k, _p(self.ids), _p(self.w), _stream())

    def replay(self, rec, layer, s0, logits):
        NL, k, S = rec.shape
        # ids and w hold (T, self.k): a record of another top_k would be
        # written past their end on the device
        if k != self.k:
            raise ValueError(f"record top_k {k} differs from the plan's k {self.k}")
        _check(rec, (NL, self.k, S), torch.int32, "record")
        _check(logits, (self.T, self.E), torch.float32, "logits")
        _call("moe_replay_load", _p(rec), NL, k, S, layer, s0, self.T, _p(logits), self.E, _p(self.ids),
              _p(self.w), _p(self.status), _stream())

    def permute(self, x):
        _check(x, (self.T, self.d), torch.bfloat16, "x")
        _call("moe_permute", _p(self.ids), self.T, self.k, self.e0, self.L, self.rcap, _p(self.counts),
              _p(self.offsets), _p(self.row_pair), _p(self.pair_row), _p(x), self.d, None, _p(self.xq),
              _p(self.xq_s), self.sflag, _p(self.ws), self.ws.numel(), _p(self.status), _stream())

    def gemm1(self, wts):
        epi = ops.EPI_SWIGLU_Q8_SAVE if self.gu is not None else ops.EPI_SWIGLU_Q8
        thin = ops.GEMM_THIN_SPLIT if self.thin_ws is not None else 0
        _call("moe_grouped_gemm_fp8", _p(self.xq), _p(self.xq_s), _p(wts["w13q"]), _p(wts["w13s"]),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, 2 * self.f, self.d, epi | self.gflag | thin, None,
              _p(self.hq), _p(self.hq_s), _p(self.gu), None, _p(self.thin_ws), None, _stream())

    def gemm2(self, wts):
        _call("moe_grouped_gemm_fp8", _p(self.hq), _p(self.hq_s), _p(wts["w2q"]), _p(wts["w2s"]),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, self.d, self.f, ops.EPI_STORE_BF16 | self.gflag,
              None,
              _p(self.Y), None, None, None, None, None, _stream())

    def combine(self):
        _call("moe_unpermute_combine", _p(self.Y), _p(self.pair_row), _p(self.w), self.T, self.k, self.d,
              self.rcap, _p(self.y), _stream())

    STAGES = ("route", "permute", "gemm1", "gemm2", "combine")

    def forward(self, x, logits, wts, replay=None, events=None):
        """One forward pass.  replay = (rec, layer, s0) replays recorded ids.
        events: optional dict name -> (start, end) torch.cuda.Event pairs."""
        def rec(name, fn, *a):
            if events is not None and name in events:
                events[name][0].record()
                fn(*a)
                events[name][1].record()
            else:
                fn(*a)
        if replay is None:
            rec("route", self.route, logits)
        else:
            rec("route", self.replay, replay[0], replay[1], replay[2], logits)
        rec("permute", self.permute, x)
        rec("gemm1", self.gemm1, wts)
        rec("gemm2", self.gemm2, wts)
        rec("combine", self.combine)
        return self.y


    def capture(self, x, logits, wts, replay=None, warmup=1):
        """Capture one ``forward`` over these exact buffers into a HIP graph
        (torch.cuda.CUDAGraph).  Every stage is a kernel launch on the current
        stream with no allocation, host synchronisation or memset, so the whole
        pass is capturable; graph.replay() reruns it on whatever x, logits and
        weights the buffers hold at that time, without per-launch host cost.
        ``warmup`` eager passes run first on the capture's side stream."""
        return capture_graph(lambda: self.forward(x, logits, wts, replay=replay), warmup)


def capture_graph(fn, warmup=1):
    """Record the launches ``fn`` issues on the current stream into a HIP graph
    (torch.cuda.CUDAGraph), after ``warmup`` eager calls on a side stream.  fn
    must only launch library kernels on preallocated buffers: no allocation,
    host synchronisation or memset."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


class TrainPlan(ForwardPlan):
    """Device buffers for one forward + backward pass of T tokens.

    Backward ("RL at 1T scale", section "FP8 Training": every backward GEMM operand
    is block-quantised along that GEMM's contraction axis):
      combine backward -> dY 1x128 and 128x1 (transposed) FP8, gate partials
      dgrad GEMM through W2 (fp32 dH) -> SwiGLU backward -> [dG, dU] 1x128 and
      128x1, recomputed H 128x1;  dgrad GEMM through W13 -> dX -> unpermute-sum dx
      (x 128x1, transposed, made with the forward's 1x128 copy);  wgrad GEMMs
      dW2 = dY^T H, dW13 = [dG, dU]^T X
      softmax-over-selection backward -> d_logits."""

    def __init__(self, T, d, f, E, L, k, e0=0, device="cuda", pow2=False, mxfp4=False):
        super().__init__(T, d, f, E, L, k, e0=e0, device=device, save_gu=True, pow2=pow2, mxfp4=mxfp4)
        # FP8 weights with d, f multiples of 256: the dgrad products read the
        # forward weights [out, in] as their [K, N] operand, so no transposed
        # copy is made; otherwise (MXFP4, or other shapes) they read the copies
        # quantize_weights(transpose=True) writes
        self.weights_kn = not mxfp4 and d % 256 == 0 and f % 256 == 0
        self.transpose_weights = not self.weights_kn
        dv = device
        f32, u8, b16 = torch.float32, torch.uint8, torch.bfloat16
        R = self.rcap
        self.dyq = torch.empty((R, d), dtype=u8, device=dv)
        self.dyq_s = torch.empty((d // 128, R), dtype=f32, device=dv)
        self.d_gate = torch.empty((T, k), dtype=f32, device=dv)
        self.dyqT = torch.empty((R // 128, d, 128), dtype=u8, device=dv)  # block-transposed
        self.dyqT_s = torch.empty((R // 128, d), dtype=f32, device=dv)  # token-block-major
        self.gate_part = torch.empty((R, ops.GATE_PARTS), dtype=f32, device=dv)
        self.dH = torch.empty((R, f), dtype=f32, device=dv)
        self.sb = dict(dgu_q=torch.empty((R, 2 * f), dtype=u8, device=dv),
                       dgu_s=torch.empty((2 * f // 128, R), dtype=f32, device=dv),
                       dgu_qT=torch.empty((R // 128, 2 * f, 128), dtype=u8, device=dv),
                       dgu_sT=torch.empty((R // 128, 2 * f), dtype=f32, device=dv),
                       h_qT=torch.empty((R // 128, f, 128), dtype=u8, device=dv),
                       h_sT=torch.empty((R // 128, f), dtype=f32, device=dv))
        self.dX = torch.empty((R, d), dtype=b16, device=dv)
        self.dx = torch.empty((T, d), dtype=b16, device=dv)
        self.xqT = torch.empty((R // 128, d, 128), dtype=u8, device=dv)
        self.xqT_s = torch.empty((R // 128, d), dtype=f32, device=dv)
        self.dW2 = torch.empty((L, d, f), dtype=b16, device=dv)
        self.dW13 = torch.empty((L, 2 * f, d), dtype=b16, device=dv)
        self.d_logits = torch.empty((T, E), dtype=f32, device=dv)

    def permute(self, x):
        """Index kernels, then x's rows quantised 1x128 (GEMM1) and 128x1
        (the dW13 product) from one read."""
        _check(x, (self.T, self.d), torch.bfloat16, "x")
        _call("moe_permute", _p(self.ids), self.T, self.k, self.e0, self.L, self.rcap, _p(self.counts),
              _p(self.offsets), _p(self.row_pair), _p(self.pair_row), None, self.d, None, None, None, self.sflag,
              _p(self.ws), self.ws.numel(), _p(self.status), _stream())
        _call("moe_quant_fp8_rows_both", _p(x), None, _p(self.row_pair), _p(self.offsets), self.T, self.L, self.rcap,
              self.k, self.d, _p(self.xq), _p(self.xq_s), _p(self.xqT), _p(self.xqT_s), self.sflag, _stream())

    def combine_bwd(self, dy):
        """dY = w * dy on the grouped rows, 1x128 and 128x1 (transposed), and the
        gate partials, from one pass over dy and Y."""
        _check(dy, (self.T, self.d), torch.bfloat16, "dy")
        _call("moe_combine_backward_rows", _p(dy), _p(self.Y), _p(self.w), _p(self.row_pair), _p(self.offsets),
              self.T, self.L, self.rcap, self.k, self.d, _p(self.dyq), _p(self.dyq_s), _p(self.dyqT), _p(self.dyqT_s),
              _p(self.gate_part), self.sflag, _stream())

    def _dgrad_weights(self, wts, name):
        if self.weights_kn:
            return wts[name + "q"], wts[name + "s"], ops.GEMM_B_KN
        return wts[name + "qT"], wts[name + "sT"], 0

    def dgrad2(self, wts):
        b, b_s, kn = self._dgrad_weights(wts, "w2")
        _call("moe_grouped_gemm_fp8", _p(self.dyq), _p(self.dyq_s), _p(b), _p(b_s),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, self.f, self.d,
              ops.EPI_STORE_F32 | self.gflag | kn, None,
              _p(self.dH), None, None, None, None, None, _stream())

    def swiglu_bwd(self):
        s = self.sb
        _call("moe_swiglu_backward", _p(self.dH), _p(self.gu), _p(self.row_pair), _p(self.offsets), self.L,
              self.rcap, self.f, _p(s["dgu_q"]), _p(s["dgu_s"]), _p(s["dgu_qT"]), _p(s["dgu_sT"]),
              _p(s["h_qT"]), _p(s["h_sT"]), None, None, self.sflag, _stream())

    def dgrad1(self, wts):
        b, b_s, kn = self._dgrad_weights(wts, "w13")
        _call("moe_grouped_gemm_fp8", _p(self.sb["dgu_q"]), _p(self.sb["dgu_s"]), _p(b), _p(b_s),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, self.d, 2 * self.f,
              ops.EPI_STORE_BF16 | self.gflag | kn, None, _p(self.dX), None, None, None, None, None, _stream())

    def unpermute(self):
        _call("moe_unpermute_combine", _p(self.dX), _p(self.pair_row), None, self.T, self.k, self.d, self.rcap,
              _p(self.dx), _stream())

    def wgrad2(self):
        _call("moe_grouped_gemm_fp8_wgrad", _p(self.dyqT), _p(self.dyqT_s), _p(self.sb["h_qT"]),
              _p(self.sb["h_sT"]), _p(self.offsets), self.L, self.rcap, self.d, self.f, _p(self.dW2), self.sflag,
              _stream())

    def wgrad13(self):
        _call("moe_grouped_gemm_fp8_wgrad", _p(self.sb["dgu_qT"]), _p(self.sb["dgu_sT"]), _p(self.xqT),
              _p(self.xqT_s), _p(self.offsets), self.L, self.rcap, 2 * self.f, self.d, _p(self.dW13), self.sflag,
              _stream())

    def gate_bwd(self):
        _call("moe_gate_backward_parts", _p(self.gate_part), _p(self.pair_row), self.rcap, self.d, _p(self.w),
              _p(self.ids), self.T, self.k, self.E, _p(self.d_gate), _p(self.d_logits), _stream())

    BWD_STAGES = ("combine_bwd", "dgrad2", "swiglu_bwd", "dgrad1", "unpermute", "wgrad2", "wgrad13", "gate_bwd")

    def backward(self, x, dy, wts, events=None):
        """Backward of the last ``forward`` for upstream gradient dy [T, d] bf16;
        wts must hold the transposed weight copies (quantize_weights(transpose=True))
        when ``self.transpose_weights``."""
        def rec(name, fn, *a):
            if events is not None and name in events:
                events[name][0].record()
                fn(*a)
                events[name][1].record()
            else:
                fn(*a)
        rec("combine_bwd", self.combine_bwd, dy)
        rec("dgrad2", self.dgrad2, wts)
        rec("swiglu_bwd", self.swiglu_bwd)
        rec("dgrad1", self.dgrad1, wts)
        rec("unpermute", self.unpermute)
        rec("wgrad2", self.wgrad2)
        rec("wgrad13", self.wgrad13)
        rec("gate_bwd", self.gate_bwd)
        return self.dx, self.dW13, self.dW2, self.d_logits
