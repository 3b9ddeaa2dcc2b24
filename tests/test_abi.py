"""CPU checks of the C ABI: the built library loads without a GPU, exports every
function include/moe_mi355x.h declares, and rejects bad arguments synchronously
(before any HIP call, so these run on a machine with no GPU)."""

import ctypes
import os
import re

import pytest

from moe_expert_layer_r3_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="library not built")


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\s*\*)\s*(moe_\w+)\s*\(", txt, re.M)))


def test_header_and_binding_agree():
    assert declared() == sorted(ops.exported_symbols())


def test_every_declared_symbol_exported():
    lib = ctypes.CDLL(ops.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def test_row_cap():
    assert ops.row_cap(8192, 8, 32) == (8192 * 8 + 32 * 127 + 127) // 128 * 128
    assert ops.row_cap(128, 2, 8) == 128 * 2 + 8 * 127 + 8 and ops.row_cap(128, 2, 8) % 128 == 0
    assert ops.row_cap(10, 8, 4) % 128 == 0 and ops.row_cap(10, 8, 4) >= 10 * 4
    assert ops.row_cap(-1, 2, 2) == -1


P = ctypes.c_void_p
FAKE = P(0x1000)   # never dereferenced: validation fails before any HIP call


def _rc(name, *args):
    rc = getattr(ops.lib(), name)(*args)
    return rc, ops.last_error()


def test_topk_validation():
    rc, msg = _rc("moe_route_topk", FAKE, 10, 1025, 2, FAKE, FAKE, None)
    assert rc == -2 and "E=1025" in msg
    rc, _ = _rc("moe_route_topk", FAKE, 10, 8, 9, FAKE, FAKE, None)
    assert rc == -2
    rc, _ = _rc("moe_route_topk", FAKE, 10, 8, 17, FAKE, FAKE, None)
    assert rc == -2
    rc, _ = _rc("moe_route_topk", None, 10, 8, 2, FAKE, FAKE, None)
    assert rc == -1
    assert _rc("moe_route_topk", None, 0, 8, 2, None, None, None)[0] == 0      # T = 0: no-op


def test_capture_and_replay_validation():
    rc, _ = _rc("moe_route_topk_capture", FAKE, 10, 8, 2, FAKE, FAKE, None, 4, 100, 0, 0, None)
    assert rc == -1
    rc, _ = _rc("moe_route_topk_capture", FAKE, 10, 8, 2, FAKE, FAKE, FAKE, 4, 100, 4, 0, None)
    assert rc == -2
    rc, _ = _rc("moe_route_topk_capture", FAKE, 10, 8, 2, FAKE, FAKE, FAKE, 4, 100, 0, 95, None)
    assert rc == -2
    rc, _ = _rc("moe_replay_load", FAKE, 4, 8, 100, 0, 95, 10, FAKE, 256, FAKE, FAKE, None, None)
    assert rc == -2
    rc, _ = _rc("moe_replay_load", FAKE, 4, 8, 100, -1, 0, 10, FAKE, 256, FAKE, FAKE, None, None)
    assert rc == -2
    rc, _ = _rc("moe_replay_load", None, 4, 8, 100, 0, 0, 10, FAKE, 256, FAKE, FAKE, None, None)
    assert rc == -1


def test_permute_validation():
    n = ctypes.c_size_t(0)
    assert ops.lib().moe_permute_workspace(8192, 8, 32, ctypes.byref(n)) == 0 and n.value > 0
    args = dict(ids=FAKE, T=100, k=2, e0=0, L=8, rcap=512, counts=FAKE, offsets=FAKE, row_pair=FAKE,
                pair_row=FAKE, x=None, d=0, xp=None, xq=None, xs=None, qf=0, ws=FAKE, wsb=1 << 20, st=None,
                s=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return _rc("moe_permute", *a.values())[0]

    assert call(rcap=500) == -2                   # not a multiple of 128
    assert call(L=0) == -2 and call(L=1025) == -2
    assert call(wsb=4) == -4                      # workspace too small
    assert call(counts=None) == -1
    assert call(x=FAKE, d=100, xq=FAKE, xs=FAKE) == -2
    assert call(x=FAKE, d=128) == -1              # x without an output
    assert call(xq=FAKE, xs=FAKE) == -1           # output without x
    assert call(qf=1) == -3 and call(qf=0x101) == -3  # unknown quant flags


def test_quant_validation():
    L = "moe_quant_fp8"
    assert _rc(L, FAKE, 2, 1, 4, 100, 100, 0, FAKE, FAKE, None, None, None)[0] == -3   # bad src type
    assert _rc(L, FAKE, 0, 1, 4, 100, 100, 0, FAKE, FAKE, None, None, None)[0] == -2   # cols % 128
    assert _rc(L, FAKE, 0, 1, 100, 128, 128, 1, FAKE, FAKE, None, None, None)[0] == -2  # rows % 128
    assert _rc(L, FAKE, 0, 1, 128, 128, 128, 0, FAKE, FAKE, FAKE, FAKE, None)[0] == -3  # qT for 1x128
    assert _rc(L, None, 0, 1, 128, 128, 128, 0, FAKE, FAKE, None, None, None)[0] == -1
    assert _rc(L, FAKE, 0, 1, 128, 128, 64, 0, FAKE, FAKE, None, None, None)[0] == -2   # ld < cols
    assert _rc(L, FAKE, 0, 1, 128, 128, 128, 0x102, FAKE, FAKE, None, None, None)[0] == -3  # unknown tile
    assert _rc(L, FAKE, 0, 1, 128, 128, 128, 0x200, FAKE, FAKE, None, None, None)[0] == -3  # unknown flag
    R = "moe_quant_fp8_rows_t"
    assert _rc(R, FAKE, None, FAKE, FAKE, 8, 200, 2, 128, FAKE, FAKE, 0, None)[0] == -2
    assert _rc(R, FAKE, None, FAKE, FAKE, 8, 256, 2, 100, FAKE, FAKE, 0, None)[0] == -2
    assert _rc(R, FAKE, None, FAKE, FAKE, 8, 256, 2, 128, FAKE, FAKE, 1, None)[0] == -3   # unknown flags


def test_gemm_validation():
    G = "moe_grouped_gemm_fp8"
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 512, 256, 0, None, FAKE, None, None, None, None, None,
            None]

    def call(**idx):
        a = list(base)
        for i, v in idx.items():
            a[int(i[1:])] = v
        return _rc(G, *a)[0]

    assert call(a8=100) == -2            # N % 128
    assert call(a9=100) == -2            # K % 128
    assert call(a7=1000) == -2           # row_cap % 128
    assert call(a6=0) == -2
    assert call(a10=9) == -3             # unknown epilogue
    assert call(a10=0x109) == -3 and call(a10=0x200) == -3  # unknown epilogue with / without POW2
    assert call(a10=0x101) == -1         # SWIGLU_Q8 | POW2 without out_s
    assert call(a10=1) == -1             # SWIGLU_Q8 without out_s
    assert call(a10=1, a8=384, a13=FAKE) == -2    # SwiGLU needs N % 256
    assert call(a0=None) == -1
    # the 128 x 256 tile flag is recognised: the same argument checks still apply
    assert call(a10=0x400, a8=100) == -2 and call(a10=0x401) == -1 and call(a10=0x409) == -3
    assert ops.GEMM_TILE128 == 0x400
    # [K, N] weights: store epilogues with FP8 weights and 256 x 256 tiles only
    assert ops.GEMM_B_KN == 0x800
    assert call(a10=0x800, a8=384) == -3            # N % 256
    assert call(a10=0x801, a13=FAKE) == -3          # SwiGLU epilogue
    assert call(a10=0xC00) == -3                    # with the 128 x 256 tile
    assert call(a10=0xB00) == -3                    # MXFP4 weights
    assert call(a10=0x803, a0=None) == -1           # accepted flags; the NULL check follows


def test_combine_validation():
    assert _rc("moe_unpermute_combine", FAKE, FAKE, FAKE, 10, 17, 128, 256, FAKE, None)[0] == -2
    assert _rc("moe_unpermute_combine", FAKE, FAKE, FAKE, 10, 2, 100, 256, FAKE, None)[0] == -2
    assert _rc("moe_unpermute_combine", FAKE, None, FAKE, 10, 2, 128, 256, FAKE, None)[0] == -1
    assert _rc("moe_combine_backward", FAKE, FAKE, FAKE, FAKE, 10, 2, 128, 256, FAKE, None, FAKE, 0, None)[0] == -1
    assert _rc("moe_combine_backward", FAKE, FAKE, FAKE, FAKE, 10, 2, 128, 256, FAKE, FAKE, FAKE, 3, None)[0] == -3
    assert _rc("moe_gate_backward", FAKE, FAKE, FAKE, 10, 2, 2000, FAKE, None)[0] == -2
    R = "moe_combine_backward_rows"
    ok = [FAKE] * 5 + [100, 8, 1024, 2, 256] + [FAKE] * 5
    assert _rc(R, *ok, 0x200, None)[0] == -3                                       # unknown flags
    bad = list(ok)
    bad[9] = 200
    assert _rc(R, *bad, 0, None)[0] == -2                                          # d % 128
    bad = list(ok)
    bad[7] = 1000
    assert _rc(R, *bad, 0, None)[0] == -2                                          # row_cap % 128
    bad = list(ok)
    bad[7], bad[9] = 1 << 20, 4096
    assert _rc(R, *bad, 0, None)[0] == -2                                          # row_cap * d >= 2^31
    bad = list(ok)
    bad[14] = None
    assert _rc(R, *bad, 0x100, None)[0] == -1                                      # gate_part NULL
    B = "moe_quant_fp8_rows_both"
    okb = [FAKE, None, FAKE, FAKE, 100, 8, 1024, 2, 256, FAKE, FAKE, FAKE, FAKE]
    assert _rc(B, *okb, 0x200, None)[0] == -3                                      # unknown flags
    bad = list(okb)
    bad[8] = 200
    assert _rc(B, *bad, 0, None)[0] == -2                                          # cols % 128
    bad = list(okb)
    bad[11] = None
    assert _rc(B, *bad, 0, None)[0] == -1                                          # qT NULL
    GP = "moe_gate_backward_parts"
    assert _rc(GP, FAKE, FAKE, 1024, 200, FAKE, FAKE, 10, 2, 64, FAKE, FAKE, None)[0] == -2   # d % 128
    assert _rc(GP, FAKE, FAKE, 1024, 256, FAKE, FAKE, 10, 17, 64, FAKE, FAKE, None)[0] == -2  # k
    assert _rc(GP, FAKE, None, 1024, 256, FAKE, FAKE, 10, 2, 64, FAKE, FAKE, None)[0] == -1


def test_backward_validation():
    W = "moe_grouped_gemm_fp8_wgrad"
    assert _rc(W, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 256, 512, FAKE, 1, None)[0] == -3      # unknown flags
    assert _rc(W, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 200, 512, FAKE, 0, None)[0] == -2      # M % 128
    assert _rc(W, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1000, 256, 512, FAKE, 0x100, None)[0] == -2  # row_cap % 128
    assert _rc(W, FAKE, None, FAKE, FAKE, FAKE, 8, 1024, 256, 512, FAKE, 0x100, None)[0] == -1
    S = "moe_swiglu_backward"
    ok = [FAKE] * 4 + [8, 1024, 256] + [FAKE] * 6 + [None, None]
    assert _rc(S, *ok, 0x200, None)[0] == -3                                                  # unknown flags
    bad_f = list(ok)
    bad_f[6] = 100
    assert _rc(S, *bad_f, 0, None)[0] == -2                                                   # f % 128
    no_h = list(ok)
    no_h[11] = None
    assert _rc(S, *no_h, 0x100, None)[0] == -1


def test_mxfp4_validation():
    Q = "moe_quant_mxfp4"
    assert _rc(Q, FAKE, 1, 4, 96, 96, FAKE, FAKE, None, None, None)[0] == -2     # cols % 128
    assert _rc(Q, FAKE, 1, 4, 128, 64, FAKE, FAKE, None, None, None)[0] == -2    # ld < cols
    assert _rc(Q, None, 1, 4, 128, 128, FAKE, FAKE, None, None, None)[0] == -1
    assert _rc(Q, FAKE, 0, 4, 128, 128, None, None, None, None, None)[0] == 0    # empty: nothing to do
    assert _rc(Q, FAKE, 1, 4, 128, 128, FAKE, FAKE, FAKE, None, None)[0] == -1   # qT without scalesT
    assert _rc(Q, FAKE, 1, 100, 128, 128, FAKE, FAKE, FAKE, FAKE, None)[0] == -2  # transpose needs rows % 128
    G = "moe_grouped_gemm_fp8"
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 512, 256, 0, None, FAKE, None, None, None, None, None, None]
    args[10] = 0x200                                                # MXFP4 without POW2
    assert _rc(G, *args)[0] == -3
    args[10] = 0x301                                                # SWIGLU_Q8 | POW2 | MXFP4 without out_s
    assert _rc(G, *args)[0] == -1
