"""moe_permute_noalloc, the permutation entry point that allocates nothing (for
callers that cannot call hipMalloc: code under HIP graph capture, tight serving
loops), through the C ABI: two calls in a row, the second on a smaller input,
each bit-exact against moe_permute with a caller workspace on the same input.
The first call on the device also sets up the library's device scratch."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import routing as OR
from oracle.numerics import bf16 as obf16
from moe_expert_layer_r3_amd import ops
from gpu_util import DEV, bf16_tensor, gpu, say

pytestmark = pytest.mark.gpu

MAX_WS = 1 << 20   # MOE_PERMUTE_NOALLOC_MAX_WS


def _outputs(T, k, L, rcap, d, dev):
    poison = {torch.int32: -7, torch.uint8: 0xA5, torch.float32: -7.0}
    e = lambda shape, dt: torch.full(shape, poison[dt], dtype=dt, device=dev)
    return dict(counts=e((L,), torch.int32), offsets=e((L + 1,), torch.int32), row_pair=e((rcap,), torch.int32),
                pair_row=e((T, k), torch.int32), xq=e((rcap, d), torch.uint8), xq_s=e((d // 128, rcap), torch.float32),
                status=torch.zeros(1, dtype=torch.int32, device=dev))


def _run(noalloc, ids, e0, L, x, pow2):
    T, k = ids.shape
    d = x.shape[1]
    rcap = ops.row_cap(T, k, L)
    o = _outputs(T, k, L, rcap, d, ids.device)
    p = ops._p
    common = (p(ids), T, k, e0, L, rcap, p(o["counts"]), p(o["offsets"]), p(o["row_pair"]), p(o["pair_row"]),
              p(x), d, None, p(o["xq"]), p(o["xq_s"]), ops.SCALE_POW2 if pow2 else 0)
    if noalloc:
        ops._call("moe_permute_noalloc", *common, p(o["status"]), ops._stream())
    else:
        ws = torch.empty(ops.permute_workspace(T, k, L), dtype=torch.uint8, device=ids.device)
        ops._call("moe_permute", *common, p(ws), ws.numel(), p(o["status"]), ops._stream())
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("pow2", [False, True])
def test_permute_noalloc_matches_workspace_path(pow2):
    rng = np.random.default_rng(71 + pow2)
    # first call: the ep8 share's routing shape (8192 tokens, top-8, experts
    # 32-63 of 256 local); second call: fewer tokens, other experts, smaller d
    for T, E, k, e0, L, d in ((8192, 256, 8, 32, 32, 512), (1000, 64, 6, 8, 16, 256)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids = gpu(np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32))
        x = bf16_tensor(obf16(rng.standard_normal((T, d))))
        say(f"permute_noalloc T={T} E={E} k={k} e0={e0} L={L} d={d} pow2={pow2}")
        ref = _run(False, ids, e0, L, x, pow2)
        got = _run(True, ids, e0, L, x, pow2)
        for name in ref:
            assert torch.equal(got[name], ref[name]), name
        assert int(got["status"].item()) == 0


def test_permute_noalloc_rejects_oversize():
    """(T, k, L) whose chunk counts exceed the device scratch: MOE_ERR_WORKSPACE
    before anything is launched (the pointers are never dereferenced)."""
    fake = ctypes.c_void_p(0x1000)
    T, k, L = 1 << 20, 8, 64          # 8192 chunks x 64 experts x 4 bytes = 2 MiB
    assert ops.permute_workspace(T, k, L) > MAX_WS
    rc = ops.lib().moe_permute_noalloc(fake, T, k, 0, L, 128 * 1024, fake, fake, fake, fake, None, 0, None, None,
                                       None, 0, None, None)
    assert rc == -4                   # MOE_ERR_WORKSPACE
    assert "scratch" in ops.last_error()
