"""Thin ctypes binding of the C ABI in include/moe_mi355x.h.

Argument marshalling only: every step runs in the HIP kernels of
libmoe_mi355x.so.  Torch supplies device memory (output tensors are allocated
with torch.empty on the input's device) and the current HIP stream.  Loading
fails loudly if the library has not been built; there is no fallback path."""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

EPI_STORE_BF16, EPI_SWIGLU_Q8, EPI_SWIGLU_Q8_SAVE, EPI_STORE_F32, EPI_SWIGLU_F32 = range(5)
TILE_1x128, TILE_128x128 = 0, 1
SCALE_POW2 = 0x100  # power-of-two (UE8M0) tile scales, OR'ed into tile / epilogue
WEIGHT_MXFP4 = 0x200  # MXFP4 weights, OR'ed (with SCALE_POW2) into a GEMM epilogue
GEMM_TILE128 = 0x400  # 128 x 256 GEMM tiles instead of 256 x 256, OR'ed into a GEMM epilogue
GEMM_B_KN = 0x800     # weights given as [L, K, N] (a dgrad product on the forward weights), OR'ed likewise
GEMM_THIN_SPLIT = 0x1000  # thin last 288-row m-tiles of a SwiGLU product split along K (workspace in out3)
SRC_BF16, SRC_F32 = 0, 1
FLAG_BAD_ID, FLAG_DUP_ID, FLAG_ROW_CAP = 1, 2, 4
ROW_ALIGN = 128


class MoeError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_row_cap": (_I64, [_I64, _I32, _I32]),
    "moe_route_topk": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_route_topk_capture": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _I32, _I64, _I32, _I64, _P]),
    "moe_replay_load": (ctypes.c_int, [_P, _I32, _I32, _I64, _I32, _I64, _I64, _P, _I32, _P, _P, _P, _P]),
    "moe_permute_workspace": (ctypes.c_int, [_I64, _I32, _I32, ctypes.POINTER(_SZ)]),
    "moe_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P,
                                   _P, _I32, _P, _P, _P, _I32, _P, _SZ, _P, _P]),
    "moe_permute_noalloc": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _I64, _P, _P, _P, _P,
                                           _P, _I32, _P, _P, _P, _I32, _P, _P]),
    "moe_quant_fp8": (ctypes.c_int, [_P, _I32, _I64, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P]),
    "moe_quant_mxfp4": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "moe_quant_fp8_rows_t": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I32, _I64, _P, _P, _I32, _P]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                            _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm_thin_workspace": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "moe_grouped_gemm_fp8_wgrad": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _I32, _P]),
    "moe_swiglu_backward": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _I32, _P]),
    "moe_unpermute_combine": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I64, _P, _P]),
    "moe_combine_backward": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I32, _I64, _P, _P, _P, _I32, _P]),
    "moe_gate_backward": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "moe_combine_backward_rows": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I32, _I64, _I32, _I32, _P, _P, _P, _P,
                                                 _P, _I32, _P]),
    "moe_gate_backward_parts": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_quant_fp8_rows_both": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I64, _I32, _I32, _P, _P, _P, _P, _I32,
                                               _P]),
}

GATE_PARTS = 16  # MOE_GATE_PARTS


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python moe_expert_layer_r3_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def exported_symbols():
    return list(_SIGS)


def last_error():
    return lib().moe_last_error().decode()


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MoeError(name, rc, last_error())


def _flag(pow2):
    return SCALE_POW2 if pow2 else 0


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    return t.device


def _contig(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def row_cap(T, k, L):
    return int(lib().moe_row_cap(T, k, L))


# ---------------------------------------------------------------- routing

def route_topk(logits, k, capture=None):
    """logits fp32 [T, E] -> (ids int32 [T, k], w fp32 [T, k]).

    capture = (rec [NL, k, S] int32, layer, s0) also records the ids."""
    _contig(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = _dev(logits)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if capture is None:
        _call("moe_route_topk", _p(logits), T, E, k, _p(ids), _p(w), _stream(dev))
    else:
        rec, layer, s0 = capture
        _contig(rec, torch.int32, "rec")
        NL, kk, S = rec.shape
        if kk != k:
            raise ValueError("record top_k differs from k")
        _call("moe_route_topk_capture", _p(logits), T, E, k, _p(ids), _p(w), _p(rec), NL, S, layer, s0,
              _stream(dev))
    return ids, w


def replay_load(rec, layer, s0, logits, status=None):
    """Router Replay: ids = rec[layer, :, s0:s0+T].T, gates from logits [T, E]."""
    _contig(rec, torch.int32, "rec")
    _contig(logits, torch.float32, "logits")
    NL, k, S = rec.shape
    T, E = logits.shape
    dev = _dev(logits)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_replay_load", _p(rec), NL, k, S, layer, s0, T, _p(logits), E, _p(ids), _p(w), _p(status),
          _stream(dev))
    return ids, w


def gate_backward(d_gate, w, ids, E):
    T, k = ids.shape
    out = torch.empty((T, E), dtype=torch.float32, device=_dev(ids))
    _call("moe_gate_backward", _p(d_gate), _p(w), _p(ids), T, k, E, _p(out), _stream(ids.device))
    return out


def gate_backward_parts(gate_part, pair_row, rcap, d, w, ids, E):
    """(d_gate [T, k], d_logits [T, E]) from the partials of combine_backward_rows."""
    T, k = ids.shape
    dev = _dev(ids)
    d_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    out = torch.empty((T, E), dtype=torch.float32, device=dev)
    _call("moe_gate_backward_parts", _p(gate_part), _p(pair_row), rcap, d, _p(w), _p(ids), T, k, E, _p(d_gate),
          _p(out), _stream(dev))
    return d_gate, out


# ---------------------------------------------------------------- dispatch

def permute_workspace(T, k, L):
    n = _SZ(0)
    _call("moe_permute_workspace", T, k, L, ctypes.byref(n))
    return n.value


def thin_workspace(L, N, K):
    """Bytes of the workspace of a SwiGLU product with GEMM_THIN_SPLIT."""
    n = _SZ(0)
    _call("moe_grouped_gemm_thin_workspace", L, N, K, ctypes.byref(n))
    return n.value


def permute(ids, e0, L, rcap=None, x=None, x_perm=False, quant=True, status=None, ws=None, pow2=False):
    """Expert-grouped permutation (+ optional fused gather / 1x128 quant of x,
    with power-of-two scales when pow2).

    Returns a dict with counts, offsets, row_pair, pair_row, row_cap and, when x
    is given, x_perm (bf16) and/or xq (u8) + xq_s (fp32)."""
    _contig(ids, torch.int32, "ids")
    T, k = ids.shape
    dev = _dev(ids)
    rcap = row_cap(T, k, L) if rcap is None else rcap
    counts = torch.empty(L, dtype=torch.int32, device=dev)
    offsets = torch.empty(L + 1, dtype=torch.int32, device=dev)
    row_pair = torch.empty(max(rcap, 1), dtype=torch.int32, device=dev)
    pair_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(permute_workspace(T, k, L), dtype=torch.uint8, device=dev)
    out = dict(counts=counts, offsets=offsets, row_pair=row_pair, pair_row=pair_row, row_cap=rcap)
    xp = xq = xs = None
    d = 0
    if x is not None:
        _contig(x, torch.bfloat16, "x")
        d = x.shape[1]
        if x_perm:
            xp = torch.empty((rcap, d), dtype=torch.bfloat16, device=dev)
        if quant:
            xq = torch.empty((rcap, d), dtype=torch.uint8, device=dev)
            xs = torch.empty((d // 128, rcap), dtype=torch.float32, device=dev)  # K-block-major
    _call("moe_permute", _p(ids), T, k, e0, L, rcap, _p(counts), _p(offsets), _p(row_pair), _p(pair_row),
          _p(x), d, _p(xp), _p(xq), _p(xs), _flag(pow2), _p(ws), ws.numel(), _p(status),
          _stream(dev))
    out.update(x_perm=xp, xq=xq, xq_s=xs)
    return out


# ---------------------------------------------------------------- quantisation

def quant_fp8(src, tile=TILE_1x128, groups=1, transpose=False, pow2=False):
    """Quantise src ([rows, cols] or [groups, rows, cols], bf16 or fp32), with
    power-of-two scales when pow2.

    Returns (q, s) or, for 128x128 with transpose=True, (q, s, qT, sT)."""
    src_type = {torch.bfloat16: SRC_BF16, torch.float32: SRC_F32}[src.dtype]
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    dev = _dev(src)
    if src.dim() == 3:
        groups, rows, cols = src.shape
    else:
        rows, cols = src.shape
        rows //= groups
    if tile == TILE_1x128:
        q = torch.empty((groups * rows, cols), dtype=torch.uint8, device=dev)
        s = torch.empty((groups * rows, cols // 128), dtype=torch.float32, device=dev)
        qT = sT = None
    else:
        q = torch.empty((groups, rows, cols), dtype=torch.uint8, device=dev)
        s = torch.empty((groups, rows // 128, cols // 128), dtype=torch.float32, device=dev)
        qT = torch.empty((groups, cols, rows), dtype=torch.uint8, device=dev) if transpose else None
        sT = torch.empty((groups, cols // 128, rows // 128), dtype=torch.float32, device=dev) if transpose else None
    _call("moe_quant_fp8", _p(src), src_type, groups, rows, cols, cols, tile | _flag(pow2), _p(q), _p(s), _p(qT), _p(sT),
          _stream(dev))
    if tile == TILE_128x128 and transpose:
        return q, s, qT, sT
    if tile == TILE_1x128 and src.dim() == 3:
        return q.view(groups, rows, cols), s.view(groups, rows, cols // 128)
    return q, s


def quant_mxfp4(src, transpose=False):
    """MXFP4 of bf16 src [G, N, K] (or [N, K]) along K: (q [G, K/128, N, 64] u8
    packed E2M1, scales [G, K/128, N, 4] u8 E8M0 codes), both K-block-major;
    with transpose also the transpose's along N: qT [G, N/128, K, 64], sT
    [G, N/128, K, 4]."""
    _contig(src, torch.bfloat16, "src")
    dev = _dev(src)
    G, N, K = src.shape if src.dim() == 3 else (1,) + tuple(src.shape)
    q = torch.empty((G, K // 128, N, 64), dtype=torch.uint8, device=dev)
    s = torch.empty((G, K // 128, N, 4), dtype=torch.uint8, device=dev)
    qT = torch.empty((G, N // 128, K, 64), dtype=torch.uint8, device=dev) if transpose else None
    sT = torch.empty((G, N // 128, K, 4), dtype=torch.uint8, device=dev) if transpose else None
    _call("moe_quant_mxfp4", _p(src), G, N, K, K, _p(q), _p(s), _p(qT), _p(sT), _stream(dev))
    return (q, s, qT, sT) if transpose else (q, s)


def mx_scales_rows(s):
    """[G, K/128, N, 4] K-block-major MXFP4 scales as numpy [G, N, K/32]."""
    G, kb, N, _ = s.shape
    return s.detach().cpu().numpy().transpose(0, 2, 1, 3).reshape(G, N, kb * 4)


def mx_codes_rows(q):
    """[G, K/128, N, 64] K-block-major packed MXFP4 codes as numpy [G, N, K/2]."""
    G, kb, N, _ = q.shape
    return q.detach().cpu().numpy().transpose(0, 2, 1, 3).reshape(G, N, kb * 64)


def untile_t(qT):
    """[cols, rcap] view (a copy) of a block-transposed operand [rcap/128, cols, 128]."""
    nb, cols, _ = qT.shape
    return qT.permute(1, 0, 2).reshape(cols, nb * 128)


def tile_t(q):
    """Block-transposed layout [rcap/128, cols, 128] of a numpy [cols, rcap] array."""
    cols, r = q.shape
    return np.ascontiguousarray(q.reshape(cols, r // 128, 128).transpose(1, 0, 2))


def quant_rows_t(src, w, row_pair, offsets, L, rcap, k, pow2=False):
    """128x1 quantisation along the expert-grouped rows (gathered from src [T, cols]
    via row_pair, optionally scaled by w), transposed: (qT [rcap/128, cols, 128]
    block-transposed, sT [rcap/128, cols])."""
    _contig(src, torch.bfloat16, "src")
    cols = src.shape[1]
    dev = _dev(src)
    qT = torch.empty((rcap // 128, cols, 128), dtype=torch.uint8, device=dev)
    sT = torch.empty((rcap // 128, cols), dtype=torch.float32, device=dev)  # token-block-major
    _call("moe_quant_fp8_rows_t", _p(src), _p(w), _p(row_pair), _p(offsets), L, rcap, k, cols, _p(qT), _p(sT),
          _flag(pow2), _stream(dev))
    return qT, sT


# ---------------------------------------------------------------- GEMMs

def grouped_gemm(a, a_s, b, b_s, counts, offsets, epilogue=EPI_STORE_BF16, epi_in=None, rcap=None, pow2=False,
                 mxfp4=False, tile128=False, b_kn=False, thin_ws=None):
    """Per-expert blockwise-scaled FP8 GEMM over the expert-grouped rows.

    a [rcap, K] u8, a_s [K/128, rcap]; b [L, N, K] u8, b_s [L, N/128, K/128].
    pow2: every scale is a power of two, applied by the MFMA as E8M0 (the
    SwiGLU epilogues then also quantise h with power-of-two scales).
    mxfp4: b [L, K/128, N, 64] and b_s [L, K/128, N, 4] from quant_mxfp4 (implies pow2).
    tile128: 128 x 256 block tiles instead of 256 x 256 (N % 256 == 0).
    b_kn: b [L, K, N], b_s [L, K/128, N/128] (the forward weights of a dgrad
    product, read without a transposed copy; FP8, store epilogues, N % 256 == 0).
    Returns the epilogue's outputs: STORE_BF16 -> y; STORE_F32 -> acc;
    SWIGLU_Q8 -> (hq, hq_s); SWIGLU_Q8_SAVE -> (hq, hq_s, gu);
    SWIGLU_F32 -> h.
    thin_ws (SwiGLU epilogues, FP8 weights, 288-row tiles): a device buffer of
    thin_workspace(L, N, K) bytes; thin last m-tiles (at most 32 rows) are then
    computed split along K."""
    rcap = a.shape[0] if rcap is None else rcap
    if mxfp4:
        L, kb, N, _ = b.shape
        K = kb * 128
        pow2 = True
    elif b_kn:
        L, K, N = b.shape
    else:
        L, N, K = b.shape
    dev = _dev(a)
    f = N // 2
    out = out_s = out2 = out2_s = out3 = out3_s = None
    if epilogue == EPI_STORE_BF16:
        out = torch.empty((rcap, N), dtype=torch.bfloat16, device=dev)
        res = out
    elif epilogue == EPI_STORE_F32:
        out = torch.empty((rcap, N), dtype=torch.float32, device=dev)
        res = out
    elif epilogue in (EPI_SWIGLU_Q8, EPI_SWIGLU_Q8_SAVE):
        out = torch.empty((rcap, f), dtype=torch.uint8, device=dev)
        out_s = torch.empty((f // 128, rcap), dtype=torch.float32, device=dev)  # K-block-major
        res = (out, out_s)
        if epilogue == EPI_SWIGLU_Q8_SAVE:
            out2 = torch.empty((rcap, N), dtype=torch.bfloat16, device=dev)
            res = (out, out_s, out2)
    elif epilogue == EPI_SWIGLU_F32:
        out = torch.empty((rcap, f), dtype=torch.float32, device=dev)
        res = out
    else:
        raise ValueError(f"unknown epilogue {epilogue}")
    if thin_ws is not None:
        if thin_ws.numel() * thin_ws.element_size() < thin_workspace(L, N, K):
            raise ValueError("thin_ws is smaller than thin_workspace(L, N, K)")
        out3 = thin_ws
    _call("moe_grouped_gemm_fp8", _p(a), _p(a_s), _p(b), _p(b_s), _p(counts), _p(offsets), L, rcap, N, K,
          epilogue | _flag(pow2) | (WEIGHT_MXFP4 if mxfp4 else 0) | (GEMM_TILE128 if tile128 else 0)
          | (GEMM_B_KN if b_kn else 0) | (GEMM_THIN_SPLIT if thin_ws is not None else 0), _p(epi_in), _p(out),
          _p(out_s), _p(out2), _p(out2_s), _p(out3), _p(out3_s), _stream(dev))
    return res


def grouped_gemm_wgrad(aT, aT_s, bT, bT_s, offsets, L, rcap, out=None, pow2=False, tile128=False):
    """dW [L, M, N] bf16 from the 128x1-quantised block-transposed operands
    aT [rcap/128, M, 128], bT [rcap/128, N, 128].  tile128: 128 x 256 tiles
    instead of 256 x 256 ones where M and N allow the latter."""
    M, N = aT.shape[1], bT.shape[1]
    dW = torch.empty((L, M, N), dtype=torch.bfloat16, device=_dev(aT)) if out is None else out
    _call("moe_grouped_gemm_fp8_wgrad", _p(aT), _p(aT_s), _p(bT), _p(bT_s), _p(offsets), L, rcap, M, N, _p(dW),
          _flag(pow2) | (GEMM_TILE128 if tile128 else 0), _stream(aT.device))
    return dW


def swiglu_backward(dH, gu, row_pair, offsets, L, rcap, inspect=False, out=None, pow2=False):
    """Backward through SwiGLU + FP8 re-quantisation of its results.

    dH [rcap, f] fp32, gu [rcap, 2f] bf16 (saved G, U).  Returns a dict with
    dgu_q, dgu_s (1x128), dgu_qT, dgu_sT (128x1, block-transposed), h_qT, h_sT and, when
    inspect, the fp32 dgu and h that were quantised.  ``out`` may hold
    preallocated tensors under the same names."""
    _contig(dH, torch.float32, "dH")
    _contig(gu, torch.bfloat16, "gu")
    f = dH.shape[1]
    dev = _dev(dH)
    o = {} if out is None else dict(out)
    shapes = dict(dgu_q=((rcap, 2 * f), torch.uint8), dgu_s=((2 * f // 128, rcap), torch.float32),
                  dgu_qT=((rcap // 128, 2 * f, 128), torch.uint8), dgu_sT=((rcap // 128, 2 * f), torch.float32),
                  h_qT=((rcap // 128, f, 128), torch.uint8), h_sT=((rcap // 128, f), torch.float32))
    if inspect:
        shapes.update(dgu=((rcap, 2 * f), torch.float32), h=((rcap, f), torch.float32))
    for name, (shape, dt) in shapes.items():
        if name not in o:
            o[name] = torch.empty(shape, dtype=dt, device=dev)
    _call("moe_swiglu_backward", _p(dH), _p(gu), _p(row_pair), _p(offsets), L, rcap, f,
          _p(o["dgu_q"]), _p(o["dgu_s"]), _p(o["dgu_qT"]), _p(o["dgu_sT"]), _p(o["h_qT"]), _p(o["h_sT"]),
          _p(o.get("dgu")), _p(o.get("h")), _flag(pow2), _stream(dev))
    return o


# ---------------------------------------------------------------- combine

def combine(y_perm, pair_row, w, rcap=None):
    """y [T, d] bf16 = sum over local slots of w * y_perm[pair_row] (w None: weights 1)."""
    T, k = pair_row.shape
    d = y_perm.shape[1]
    rcap = y_perm.shape[0] if rcap is None else rcap
    y = torch.empty((T, d), dtype=torch.bfloat16, device=_dev(pair_row))
    _call("moe_unpermute_combine", _p(y_perm), _p(pair_row), _p(w), T, k, d, rcap, _p(y), _stream(y.device))
    return y


def quant_rows_both(src, w, row_pair, offsets, L, rcap, k, pow2=False):
    """The expert-grouped rows of src (times w per pair if given) quantised
    1x128 and 128x1 from one read: (q [rcap, cols], q_s [cols/128, rcap],
    qT [rcap/128, cols, 128], qT_s [rcap/128, cols])."""
    _contig(src, torch.bfloat16, "src")
    cols = src.shape[1]
    dev = _dev(src)
    q = torch.empty((rcap, cols), dtype=torch.uint8, device=dev)
    qs = torch.empty((cols // 128, rcap), dtype=torch.float32, device=dev)
    qT = torch.empty((rcap // 128, cols, 128), dtype=torch.uint8, device=dev)
    qT_s = torch.empty((rcap // 128, cols), dtype=torch.float32, device=dev)
    _call("moe_quant_fp8_rows_both", _p(src), _p(w), _p(row_pair), _p(offsets), src.shape[0], L, rcap, k, cols,
          _p(q), _p(qs), _p(qT), _p(qT_s), _flag(pow2), _stream(dev))
    return q, qs, qT, qT_s


def combine_backward_rows(dy, y_perm, w, row_pair, offsets, L, rcap, k, pow2=False):
    """Both FP8 copies of dY = w * dy on the expert-grouped rows and the gate
    partials: (dyq [rcap, d], dyq_s [d/128, rcap], dyqT [rcap/128, d, 128],
    dyqT_s [rcap/128, d], gate_part [rcap, GATE_PARTS])."""
    _contig(dy, torch.bfloat16, "dy")
    d = dy.shape[1]
    dev = _dev(dy)
    dyq = torch.empty((rcap, d), dtype=torch.uint8, device=dev)
    dys = torch.empty((d // 128, rcap), dtype=torch.float32, device=dev)
    dyqT = torch.empty((rcap // 128, d, 128), dtype=torch.uint8, device=dev)
    dyqT_s = torch.empty((rcap // 128, d), dtype=torch.float32, device=dev)
    part = torch.empty((rcap, GATE_PARTS), dtype=torch.float32, device=dev)
    _call("moe_combine_backward_rows", _p(dy), _p(y_perm), _p(w), _p(row_pair), _p(offsets), dy.shape[0], L, rcap, k,
          d, _p(dyq),
          _p(dys), _p(dyqT), _p(dyqT_s), _p(part), _flag(pow2), _stream(dev))
    return dyq, dys, dyqT, dyqT_s, part


def combine_backward(dy, y_perm, pair_row, w, rcap=None, quant=True, pow2=False):
    """(dYq [rcap, d] u8, dYq_s [d/128, rcap] (K-block-major), d_gate [T, k] fp32)."""
    T, k = pair_row.shape
    d = dy.shape[1]
    rcap = y_perm.shape[0] if rcap is None else rcap
    dev = _dev(dy)
    dyq = torch.empty((rcap, d), dtype=torch.uint8, device=dev) if quant else None
    dys = torch.empty((d // 128, rcap), dtype=torch.float32, device=dev) if quant else None
    d_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_combine_backward", _p(dy), _p(y_perm), _p(pair_row), _p(w), T, k, d, rcap, _p(dyq), _p(dys),
          _p(d_gate), _flag(pow2), _stream(dev))
    return dyq, dys, d_gate
