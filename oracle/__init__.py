"""Reference oracle for the MoE expert layer (test infrastructure, not product code).

Plain, slow, CPU-only numpy implementation of what the MI355X library computes:
top-k routing or Router Replay, the expert-grouped token permutation, block-scaled
FP8 e4m3 quantisation, the blockwise-scaled grouped GEMMs with a SwiGLU between
them, the weighted combine, and the training backward.

Only the test suite, the smoke entry point and the CPU-baseline leg of the
benchmark may import this package.  The library never calls it, and it shares no
code, table or helper with the library.

Sources it follows (cited by page title and section):
  * "RL at 1T scale: a deep dive into prime-rl performance" (Prime Intellect blog,
    Chinese translation) -- sections "Router Replay" (recorded routing decisions,
    payload shaped [num_layers, top_k, seq_len], handled as an opaque tensor),
    "FP8 Training" (block-scaled FP8 as proposed by DeepSeek-V3), "Wide Expert
    Parallelism" and "Parallelism strategies / Expert Parallel" (per-layer dispatch
    and combine around experts held one set per GPU).
  * The OCP 8-bit floating point specification (E4M3FN encoding).
Every point the pages leave open is a reading listed in the design doc; each function
states which reading it takes.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_*.py (brute force, closed forms, library cross-checks,
invariants).  The only unpinned item is the layer as a whole against the pages'
own system: the pages print no worked example or value of any step.
"""

from . import numerics, routing, dispatch, blockfp8, gemm, layer  # noqa: F401
