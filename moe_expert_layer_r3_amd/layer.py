"""The MoE expert layer on one GPU's share of experts, as a sequence of C-ABI
calls on preallocated device buffers (no allocation per step).

Forward:  route (top-k, or Router Replay of recorded ids) -> permute + gather +
1x128 FP8 quant -> grouped GEMM1 with fused SwiGLU + 1x128 quant -> grouped
GEMM2 -> weighted combine.  Weights are quantised once per weight version
(128x128 tiles) by ``quantize_weights``."""

import torch

from . import ops
from .ops import _call, _p, _stream


def quantize_weights(W13, W2, transpose=False):
    """bf16 W13 [L, 2f, d], W2 [L, d, f] -> dict of FP8 codes and scales (and the
    transposed copies used by the dgrad GEMMs when ``transpose``)."""
    out = {}
    r13 = ops.quant_fp8(W13, tile=ops.TILE_128x128, transpose=transpose)
    r2 = ops.quant_fp8(W2, tile=ops.TILE_128x128, transpose=transpose)
    out["w13q"], out["w13s"] = r13[0], r13[1]
    out["w2q"], out["w2s"] = r2[0], r2[1]
    if transpose:
        out["w13qT"], out["w13sT"] = r13[2], r13[3]
        out["w2qT"], out["w2sT"] = r2[2], r2[3]
    return out


class ForwardPlan:
    """Device buffers for one forward pass of T tokens."""

    def __init__(self, T, d, f, E, L, k, e0=0, device="cuda", save_gu=False):
        self.T, self.d, self.f, self.E, self.L, self.k, self.e0 = T, d, f, E, L, k, e0
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
        self.xq_s = torch.empty((R, d // 128), dtype=f32, device=dv)
        self.hq = torch.empty((R, f), dtype=u8, device=dv)
        self.hq_s = torch.empty((R, f // 128), dtype=f32, device=dv)
        self.gu = torch.empty((R, 2 * f), dtype=b16, device=dv) if save_gu else None
        self.Y = torch.empty((R, d), dtype=b16, device=dv)
        self.y = torch.empty((T, d), dtype=b16, device=dv)

    # each stage is one C-ABI call on the current stream
    def route(self, logits):
        _call("moe_route_topk", _p(logits), self.T, self.E, self.k, _p(self.ids), _p(self.w), _stream())

    def replay(self, rec, layer, s0, logits):
        NL, k, S = rec.shape
        _call("moe_replay_load", _p(rec), NL, k, S, layer, s0, self.T, _p(logits), self.E, _p(self.ids),
              _p(self.w), _p(self.status), _stream())

    def permute(self, x):
        _call("moe_permute", _p(self.ids), self.T, self.k, self.e0, self.L, self.rcap, _p(self.counts),
              _p(self.offsets), _p(self.row_pair), _p(self.pair_row), _p(x), self.d, None, _p(self.xq),
              _p(self.xq_s), _p(self.ws), self.ws.numel(), _p(self.status), _stream())

    def gemm1(self, wts):
        epi = ops.EPI_SWIGLU_Q8_SAVE if self.gu is not None else ops.EPI_SWIGLU_Q8
        _call("moe_grouped_gemm_fp8", _p(self.xq), _p(self.xq_s), _p(wts["w13q"]), _p(wts["w13s"]),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, 2 * self.f, self.d, epi, None,
              _p(self.hq), _p(self.hq_s), _p(self.gu), None, None, None, _stream())

    def gemm2(self, wts):
        _call("moe_grouped_gemm_fp8", _p(self.hq), _p(self.hq_s), _p(wts["w2q"]), _p(wts["w2s"]),
              _p(self.counts), _p(self.offsets), self.L, self.rcap, self.d, self.f, ops.EPI_STORE_BF16, None,
              _p(self.Y), None, None, None, None, None, _stream())

    def combine(self):
        _call("moe_unpermute_combine", _p(self.Y), _p(self.pair_row), _p(self.w), self.T, self.k, self.d,
              self.rcap, _p(self.y), _stream())

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
