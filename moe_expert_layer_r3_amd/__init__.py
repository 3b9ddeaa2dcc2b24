"""MI355X-native MoE expert layer: top-k routing or Router Replay, expert-grouped
token permutation, block-scaled FP8 SwiGLU grouped GEMM and weighted combine, with
the training backward, as hand-written HIP kernels for gfx950 behind a C ABI.

Importing the package is cheap; the HIP library loads on first use of
``moe_expert_layer_r3_amd.ops``."""
