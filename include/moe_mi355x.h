/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) MoE expert-layer library.
 *
 * One Mixture-of-Experts layer on one GPU's share of experts: top-k routing or
 * Router Replay of recorded expert ids, the expert-grouped token permutation,
 * block-scaled FP8 e4m3 quantisation, an MFMA FP8 grouped GEMM with a fused
 * SwiGLU epilogue, the weighted combine, and the training backward.
 *
 * Sources (cited by page and section):
 *   [R3]  "RL at 1T scale: a deep dive into prime-rl performance", section
 *         "Router Replay": routing decisions captured at inference are replayed
 *         in the trainer; the record is shaped [num_layers, top_k, seq_len] and is
 *         handled as an opaque tensor by device ops only (no host conversion).
 *   [EP]  same page, sections "Wide Expert Parallelism" and "Parallelism
 *         strategies / Expert Parallel": each GPU holds its own experts; tokens
 *         are dispatched to them and combined back once per layer.
 *   [FP8] same page, section "FP8 Training": trainer GEMMs run in block-scaled
 *         FP8 as proposed by DeepSeek-V3 (here: 1x128 activation tiles, 128x128
 *         weight tiles, fp32 scales, e4m3 codes).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers to caller-owned memory unless stated.  The
 *     library never allocates device memory and never synchronises; every call
 *     enqueues its kernels on `stream` and returns once they are launched.
 *     Outputs are valid when the stream reaches that point; inputs must stay
 *     unchanged until then.
 *   - bf16 is passed as uint16_t bit patterns, FP8 as uint8_t OCP E4M3FN codes
 *     (bias 7, max +-448, NaN 0x7F/0xFF, no infinity), scales as fp32, indices as
 *     int32, all row-major and densely packed unless a leading dimension is given.
 *   - Argument and shape errors are detected on the host before any HIP call and
 *     return a negative moe_status; nothing is launched then.  moe_last_error()
 *     returns a thread-local message for the last failure on the calling thread.
 *   - Data-dependent problems (a replayed id out of range, a row capacity that is
 *     too small) are reported by OR-ing MOE_FLAG_* bits into the nullable device
 *     word `dev_status`; the library never clears it.  Kernels never write out of
 *     bounds on such input.
 *   - Calls are deterministic: the same inputs give bitwise-equal outputs.
 *
 * Supported shapes: hidden size d and expert FFN size f multiples of 128;
 * 1 <= top_k <= 16; 1 <= E <= 1024; local experts [e0, e0+L) inside [0, E).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL                        */
    MOE_ERR_SHAPE = -2,       /* sizes inconsistent or out of the supported range  */
    MOE_ERR_UNSUPPORTED = -3, /* a mode or combination the library does not offer  */
    MOE_ERR_WORKSPACE = -4,   /* workspace smaller than the required size          */
    MOE_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed        */
} moe_status;

enum { MOE_FLAG_BAD_ID = 1, MOE_FLAG_DUP_ID = 2, MOE_FLAG_ROW_CAP = 4 };

/* Rows of the expert-grouped layout are padded per expert to a multiple of this. */
#define MOE_ROW_ALIGN 128

/* Text of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Row capacity sufficient for any valid routing of T tokens with top_k = k onto L
 * local experts: T*min(k, L) real rows + up to 127 padding rows per expert,
 * rounded up to a multiple of 128.  Returns -1 for negative arguments. */
int64_t moe_row_cap(int64_t T, int32_t k, int32_t L);

/* ---- routing ------------------------------------------------------------- */

/* Top-k routing over fp32 router logits.
 * logits [T, E] fp32.  For each token, selects the k largest logits, ties broken
 * by the lower expert id, with IEEE comparison (-0 == +0); ids[t, 0] is the
 * largest.  Gates w[t, j] = softmax of the k selected logits (the full softmax
 * renormalised over the selection).  Logits must be finite.
 * Outputs: ids [T, k] int32, w [T, k] fp32.  T = 0 is a no-op.
 * MOE_ERR_SHAPE unless 0 <= T <= 2^33, 1 <= E <= 1024, 1 <= k <= min(16, E).  */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                   int32_t* ids, float* w, hipStream_t stream);

/* Top-k routing that also records the selection for Router Replay [R3]: as
 * moe_route_topk, and additionally writes rec[layer, j, s0 + t] = ids[t, j] into
 * the record rec [n_layers, k, seq_len] int32 (the inference-side capture).
 * Requires 0 <= layer < n_layers and s0 + T <= seq_len.                      */
int moe_route_topk_capture(const float* logits, int64_t T, int32_t E, int32_t k,
                           int32_t* ids, float* w,
                           int32_t* rec, int32_t n_layers, int64_t seq_len,
                           int32_t layer, int64_t s0, hipStream_t stream);

/* Router Replay load [R3]: replays recorded expert ids instead of recomputing
 * top-k.  rec [n_layers, k, seq_len] int32 is the recorded payload; the call
 * processes tokens s0 .. s0+T-1 of layer `layer`:
 *     ids[t, j] = rec[layer, j, s0 + t]            (verbatim, recorded slot order)
 *     w[t, :]   = softmax of logits[t, ids[t, :]]  (max shift over the k gathered)
 * logits [T, E] fp32 are the trainer's logits for those tokens.  A token with an
 * id outside [0, E) sets MOE_FLAG_BAD_ID and gets w = 0 for all slots; a token
 * with a repeated id sets MOE_FLAG_DUP_ID and keeps its computed gates.
 * dev_status may be NULL (flags are then dropped).                           */
int moe_replay_load(const int32_t* rec, int32_t n_layers, int32_t k, int64_t seq_len,
                    int32_t layer, int64_t s0, int64_t T, const float* logits, int32_t E,
                    int32_t* ids, float* w, int32_t* dev_status, hipStream_t stream);

/* ---- dispatch (local permutation) [EP] ---------------------------------- */

/* Workspace bytes moe_permute needs for T tokens, top-k k, L local experts. */
int moe_permute_workspace(int64_t T, int32_t k, int32_t L, size_t* bytes);

/* Expert-grouped permutation of the (token, slot) pairs whose expert lies in
 * [e0, e0+L).  Pair p = t*k + j, local expert le = ids[t, j] - e0.
 *   counts[e]   (int32 [L])     local pairs of expert e
 *   offsets[e]  (int32 [L+1])   offsets[0] = 0, offsets[e+1] = offsets[e] +
 *                               ceil(counts[e]/128)*128
 *   row_pair[r] (int32 [row_cap]) pair held by row r, -1 for padding rows
 *                               r < offsets[L]; entries at and past offsets[L]
 *                               are left unchanged
 *   pair_row[p] (int32 [T, k])  row of pair p, -1 for non-local pairs
 * The pairs of expert e occupy rows offsets[e] ... in ascending p (stable).
 * If offsets[L] > row_cap, MOE_FLAG_ROW_CAP is set and pairs whose row would be
 * >= row_cap get pair_row = -1 (they are dropped, nothing is written out of
 * bounds).  row_cap must be a multiple of 128; moe_row_cap() is always enough
 * for distinct ids per token.
 * Optional fused row gather (x != NULL): x [T, d] bf16.  For every real row r:
 *   x_perm[r, :] = x[t(r), :]                        (if x_perm != NULL, bf16)
 *   xq[r, :], xq_s[:, r] = 1x128 FP8 quantisation of x[t(r), :]   (if xq != NULL;
 *                          xq [row_cap, d] u8, xq_s [d/128, row_cap] fp32: scales
 *                          are stored K-block-major, the layout the GEMM reads)
 * Padding rows of x_perm / xq / xq_s are not written.
 * quant_flags: 0, or MOE_SCALE_POW2 for power-of-two xq_s scales (below).
 * ws: device workspace of at least moe_permute_workspace() bytes.            */
int moe_permute(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L,
                int64_t row_cap, int32_t* counts, int32_t* offsets,
                int32_t* row_pair, int32_t* pair_row,
                const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq, float* xq_s,
                int32_t quant_flags, void* ws, size_t ws_bytes, int32_t* dev_status,
                hipStream_t stream);

/* Largest workspace, in bytes, that moe_permute_noalloc can serve from its
 * device scratch: moe_permute_noalloc accepts (T, k, L) iff
 * moe_permute_workspace(T, k, L) <= this (e.g. T*k <= 8M pairs at L = 32). */
#define MOE_PERMUTE_NOALLOC_MAX_WS (1 << 20)

/* moe_permute without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and errors as moe_permute;
 * the workspace is a fixed device array of MOE_PERMUTE_NOALLOC_MAX_WS bytes
 * inside the library (one per GPU, held until the process ends).  Larger
 * (T, k, L) return MOE_ERR_WORKSPACE before anything is launched.  The call
 * allocates nothing; its first call on a device looks up that device's copy of
 * the array (a HIP symbol lookup, no allocation).  Every call on one GPU shares
 * the array: calls that overlap on one GPU (different streams) race and must
 * be serialised by the caller.                                               */
int moe_permute_noalloc(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L,
                        int64_t row_cap, int32_t* counts, int32_t* offsets,
                        int32_t* row_pair, int32_t* pair_row,
                        const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq, float* xq_s,
                        int32_t quant_flags, int32_t* dev_status, hipStream_t stream);

/* ---- block-scaled FP8 quantisation [FP8] -------------------------------- */

enum { MOE_TILE_1x128 = 0, MOE_TILE_128x128 = 1 };
enum { MOE_SRC_BF16 = 0, MOE_SRC_F32 = 1 };
/* OR'ed into moe_quant_fp8's tile, moe_permute's quant_flags and
 * moe_grouped_gemm_fp8's epilogue: power-of-two (UE8M0) scales.  The scale of
 * a tile with a = max(max|v|, 2^-40) is s = 2^e, e the least integer with
 * a <= 448 * 2^e, and inv = 2^-e (both exact), in place of s = a/448.  The
 * scales stay fp32 values in the same layouts; the GEMM then applies them as
 * E8M0 exponents inside the matrix instruction.                              */
enum { MOE_SCALE_POW2 = 0x100 };
/* OR'ed (with MOE_SCALE_POW2) into moe_grouped_gemm_fp8's epilogue: the weights
 * b are MXFP4 from moe_quant_mxfp4 instead of 128x128 FP8.                     */
enum { MOE_WEIGHT_MXFP4 = 0x200 };
/* OR'ed into moe_grouped_gemm_fp8's epilogue: compute with 128 x 256 block
 * tiles instead of the default 256 x 256 ones (N % 256 == 0; with
 * N % 256 != 0 the 128 x 128 tile is used either way).  The result is the same
 * up to the order of the fp32 block sums.                                     */
enum { MOE_GEMM_TILE128 = 0x400 };
/* OR'ed into moe_grouped_gemm_fp8's epilogue (STORE_BF16 or STORE_F32, FP8
 * weights, N % 256 == 0, not with MOE_GEMM_TILE128): b is [L, K, N] with b_s
 * [L, K/128, N/128], i.e. the product reads b[e, k, n] where it would read
 * b[e, n, k].  This is how a dgrad product reads the forward weights [out, in]
 * (K = out, N = in) and their moe_quant_fp8 scales without a transposed copy
 * ("RL at 1T scale", section "FP8 Training": each GEMM operand quantised along
 * its contraction axis; the 128x128 weight tiles serve both directions).    */
enum { MOE_GEMM_B_KN = 0x800 };
/* OR'ed into moe_grouped_gemm_fp8's epilogue (a SwiGLU epilogue, FP8 weights,
 * not with MOE_GEMM_TILE128): an expert whose last 288-row m-tile would hold
 * at most 32 rows gets those rows from a K-split product instead (fp32
 * partials of 4 K blocks each, summed in K order in a second launch, then the
 * same epilogue), so that no workgroup runs a whole K loop for a few rows.
 * out3 is then the caller's workspace of moe_grouped_gemm_thin_workspace
 * bytes (device memory, fp32-aligned); calls that share one workspace must
 * not overlap.  Results differ from the plain product only in the order of
 * the fp32 block sums of those rows. */
enum { MOE_GEMM_THIN_SPLIT = 0x1000 };

/* Quantise src viewed as `groups` matrices of [rows, cols] (row stride ld
 * elements, group stride rows*ld) to OCP e4m3 with one fp32 scale per tile:
 *     a = max(max|v|, 2^-40);  inv = 448 / a;  s = a / 448  (fp32, correctly
 *     rounded);  q = e4m3_rne_satfinite(fp32(v * inv))
 * tile MOE_TILE_1x128:   q [groups*rows, cols], scales [groups*rows, cols/128]
 * tile MOE_TILE_128x128: q [groups, rows, cols], scales [groups, rows/128, cols/128];
 *                        if qT != NULL also the per-group transpose
 *                        qT [groups, cols, rows] with scalesT [groups, cols/128, rows/128]
 *                        (used by the dgrad GEMMs, which read the weights transposed).
 * cols % 128 == 0; for 128x128 also rows % 128 == 0.                          */
int moe_quant_fp8(const void* src, int32_t src_type, int64_t groups, int64_t rows,
                  int64_t cols, int64_t ld, int32_t tile, uint8_t* q, float* scales,
                  uint8_t* qT, float* scalesT, hipStream_t stream);

/* MXFP4 quantisation (OCP Microscaling v1.0 FP4) of bf16 weight rows along
 * their columns (the consuming GEMM's K), for moe_grouped_gemm_fp8 with
 * MOE_WEIGHT_MXFP4 ("RL at 1T scale", section on future work: 4-bit training
 * and inference).  For every block of 32 consecutive columns of a row:
 *     E = floor(log2(max|v|)) - 2 clamped to [-127, 127] (-127 for a zero block)
 *     scales[r, c/32] = E + 127 (E8M0);  code = nearest E2M1 magnitude of
 *     |v| * 2^-E (0, 0.5, 1, 1.5, 2, 3, 4, 6; ties to the even code; above 6
 *     clamped to 6) with the sign bit of v
 *   src: groups matrices [rows, cols] bf16, row stride ld (>= cols, multiple
 *   of 8), group stride rows*ld;
 *   q [groups, cols/128, rows, 64] u8: the 128 codes of one row and 128-column
 *   block are 64 adjacent bytes (element 2b in the low nibble of byte b);
 *   scales [groups, cols/128, rows, 4] u8.  Both are K-block-major: a block's
 *   rows follow each other, the order the GEMM's K steps read.
 *   cols % 128 == 0.
 * qT, scalesT (both or neither; rows % 128 == 0): also the MXFP4 of each
 *   group's transpose [cols, rows], blocks of 32 consecutive rows, for the
 *   dgrad products: qT [groups, rows/128, cols, 64], scalesT [groups, rows/128,
 *   cols, 4] (the same layout with rows and cols exchanged); one pass reads
 *   src once for both.                                                       */
int moe_quant_mxfp4(const uint16_t* src, int64_t groups, int64_t rows, int64_t cols, int64_t ld,
                    uint8_t* q, uint8_t* scales, uint8_t* qT, uint8_t* scalesT, hipStream_t stream);

/* 128x1 quantisation along rows of the expert-grouped layout, transposed output,
 * for the wgrad GEMMs (operands re-quantised along their contraction axis, the
 * token axis).  Transposed outputs here and in moe_swiglu_backward are tiled by
 * token block ("block-transposed"): qT[b][c][i] holds row 128b + i, column c,
 * i.e. [row_cap/128, cols, 128] bytes, so that 128 columns of one token block
 * are one contiguous 16 KB piece.  Source row r is  v[r, c] = fp32(w[p] * src[p / k, c])  for the
 * pair p = row_pair[r] (w == NULL: v = src[p / k, c]); padding rows are 0.
 * Tiles are the 128-row blocks [128b, 128b+128) for 128b < offsets[L] (every
 * block lies inside one expert because segments are 128-aligned).
 *   src [T, cols] bf16;  qT [row_cap/128, cols, 128] u8 (block-transposed);
 *   sT [row_cap/128, cols] fp32 (token-block-major scales, the layout the wgrad
 *   GEMM reads).  Token blocks at and past offsets[L]/128 are left unchanged.
 * flags: 0, or MOE_SCALE_POW2 for power-of-two scales.                       */
int moe_quant_fp8_rows_t(const uint16_t* src, const float* w, const int32_t* row_pair,
                         const int32_t* offsets, int32_t L, int64_t row_cap, int32_t k,
                         int64_t cols, uint8_t* qT, float* sT, int32_t flags,
                         hipStream_t stream);

/* Both quantisations of the expert-grouped rows from one read: the rows v of
 * moe_quant_fp8_rows_t (v[r, c] = fp32(w[p] * src[p / k, c]) for p =
 * row_pair[r], w == NULL: v = src[p / k, c]) quantised
 *   1x128 along the columns:  q [row_cap, cols] u8, q_s [cols/128, row_cap] fp32
 *                             (K-block-major; padding rows not written), as the
 *                             gather of moe_permute writes xq for w == NULL
 *   128x1 along the rows:     qT, qT_s exactly as moe_quant_fp8_rows_t
 * ("RL at 1T scale", section "FP8 Training": the forward GEMM and the wgrad
 * product contract x over different axes).  Rows at and past offsets[L] are
 * not touched.  src [T, cols] bf16; cols % 128 == 0, row_cap % 128 == 0,
 * row_cap * cols and T * cols below 2^31 (MOE_ERR_SHAPE).
 * flags: 0, or MOE_SCALE_POW2 for power-of-two scales on both copies.        */
int moe_quant_fp8_rows_both(const uint16_t* src, const float* w, const int32_t* row_pair,
                            const int32_t* offsets, int64_t T, int32_t L, int64_t row_cap, int32_t k,
                            int32_t cols, uint8_t* q, float* q_s, uint8_t* qT, float* qT_s,
                            int32_t flags, hipStream_t stream);

/* ---- grouped GEMM [FP8] ------------------------------------------------- */

enum {
    MOE_EPI_STORE_BF16 = 0,      /* out  = bf16 [row_cap, N]                             */
    MOE_EPI_SWIGLU_Q8 = 1,       /* N = 2f: h = silu(G)*U (G = cols [0,f), U = [f,2f));
                                    out = hq u8 [row_cap, f], out_s = [f/128, row_cap]   */
    MOE_EPI_SWIGLU_Q8_SAVE = 2,  /* as SWIGLU_Q8, and out2 = bf16 [G, U] [row_cap, 2f]   */
    MOE_EPI_STORE_F32 = 3,       /* out  = fp32 accumulators [row_cap, N] (inspection)  */
    MOE_EPI_SWIGLU_F32 = 4       /* out  = fp32 h [row_cap, f] before quantisation
                                    (inspection of the fused quantiser's input)         */
};

/* Per-expert GEMM over the expert-grouped rows: for expert e, real rows
 * r in [offsets[e], offsets[e] + counts[e]):
 *     acc[r, n] = sum over 128-blocks c of K:
 *                 a_s[c, r] * b_s[e, n/128, c] * sum_i dec(a[r, 128c+i]) * dec(b[e, n, 128c+i])
 * accumulated in fp32, then passed through the epilogue.
 *   a [row_cap, K] e4m3, a_s [K/128, row_cap] (K-block-major: the 128 rows of a
 *   tile share contiguous scales per K block); b [L, N, K] e4m3 (weights [out, in];
 *   the dgrad products pass the transposed weights from moe_quant_fp8's qT),
 *   b_s [L, N/128, K/128].  K, N multiples of 128.  Padding rows of the outputs
 *   are not written.  Rows past row_cap are never touched.
 * epilogue | MOE_SCALE_POW2: every a_s and b_s value must be a power of two in
 *   [2^-126, 2^127] (as the MOE_SCALE_POW2 quantisers write them); the matrix
 *   instruction applies them as E8M0 exponents (any mantissa bits are
 *   ignored), and the SwiGLU epilogues quantise h with power-of-two scales.
 * epilogue | MOE_SCALE_POW2 | MOE_WEIGHT_MXFP4: b is MXFP4, b [L, K/128, N, 64]
 *   packed E2M1 and b_s (passed as float*, read as bytes) [L, K/128, N, 4]
 *   E8M0 codes, both from moe_quant_mxfp4 with groups = L, rows = N, cols = K:
 *     acc[r, n] = sum_k a_s[k/128, r] dec8(a[r, k]) * 2^(b_s[e, k/128, n, (k/32)%4] - 127) dec4(W[e, n, k])
 *   with W[e, n, k] the code in b[e, k/128, n, (k%128)/2] (low nibble for even k).
 *   (the fp4 variant exists for the forward products; the other rules hold). */
int moe_grouped_gemm_fp8(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                         const int32_t* counts, const int32_t* offsets, int32_t L,
                         int64_t row_cap, int32_t N, int32_t K, int32_t epilogue,
                         const uint16_t* epi_in, void* out, float* out_s,
                         void* out2, float* out2_s, void* out3, float* out3_s,
                         hipStream_t stream);

/* Workspace bytes for MOE_GEMM_THIN_SPLIT with L experts, N = 2f and K:
 * L * (N/256) * ceil(K/512) * 32 KB (fp32 partials of every expert's
 * n-tiles and K runs).  N % 256 == 0, K % 128 == 0 (MOE_ERR_SHAPE). */
int moe_grouped_gemm_thin_workspace(int32_t L, int32_t N, int32_t K, size_t* bytes);

/* Weight-gradient grouped GEMM: for every local expert e,
 *     dW[e][m, n] = sum over the 128-row token blocks b of e's padded segment:
 *                   aT_s[b, m] * bT_s[b, n] * sum_i dec(aT[b][m][i]) * dec(bT[b][n][i])
 * accumulated in fp32 and stored as bf16.
 *   aT [row_cap/128, M, 128] e4m3 (block-transposed), aT_s [row_cap/128, M];
 *   bT [row_cap/128, N, 128], bT_s [row_cap/128, N] (from moe_quant_fp8_rows_t
 *   or moe_swiglu_backward); dW [L, M, N] bf16.  row_cap < 2^31.
 *   An expert with no rows gets dW[e] = 0.  M, N multiples of 128.
 * flags MOE_SCALE_POW2: every aT_s and bT_s value is a power of two in
 *   [2^-126, 2^127], applied by the matrix instruction as E8M0 exponents.     */
int moe_grouped_gemm_fp8_wgrad(const uint8_t* aT, const float* aT_s, const uint8_t* bT,
                               const float* bT_s, const int32_t* offsets, int32_t L,
                               int64_t row_cap, int32_t M, int32_t N, uint16_t* dW,
                               int32_t flags, hipStream_t stream);

/* ---- SwiGLU backward [FP8] --------------------------------------------- */

/* Backward through h = silu(G) * U for the rows of the expert-grouped layout
 * ("RL at 1T scale", section "FP8 Training": every backward GEMM operand is
 * block-quantised along that GEMM's contraction axis).  With s = sigmoid(G),
 * in fp32, from dH (the dgrad GEMM through W2, MOE_EPI_STORE_F32) and the saved
 * bf16 [G, U] (MOE_EPI_SWIGLU_Q8_SAVE's out2):
 *     dG = dH * U * s * (1 + G * (1 - s)),  dU = dH * G * s,  H = G * s * U
 * Outputs (quantised as in moe_quant_fp8):
 *   dgu_q [row_cap, 2f] u8 + dgu_s [2f/128, row_cap]   1x128 tiles of [dG, dU]
 *   dgu_qT [row_cap/128, 2f, 128] u8 + dgu_sT [row_cap/128, 2f]
 *                                  128x1 tiles of [dG, dU], block-transposed
 *   h_qT [row_cap/128, f, 128] u8 + h_sT [row_cap/128, f]
 *                                  128x1 tiles of H, block-transposed
 *   (block-transposed as in moe_quant_fp8_rows_t)
 *   (scales in the layouts the GEMMs read: K-block-major, token-block-major)
 *   dgu_f32 [row_cap, 2f], h_f32 [row_cap, f]          optional (NULL = skip):
 *                                                      the fp32 values quantised
 * Padding rows (row_pair < 0) are 0 in the 128x1 tiles and are not written in
 * the row-major outputs; rows at and past offsets[L] are not touched at all.
 *   dH [row_cap, f] fp32, gu [row_cap, 2f] bf16, row_pair [row_cap]; f % 128 == 0,
 *   row_cap % 128 == 0 and row_cap / 128 <= 65535 (MOE_ERR_SHAPE otherwise).
 * flags: 0, or MOE_SCALE_POW2 for power-of-two scales on every output.        */
int moe_swiglu_backward(const float* dH, const uint16_t* gu, const int32_t* row_pair,
                        const int32_t* offsets, int32_t L, int64_t row_cap, int32_t f,
                        uint8_t* dgu_q, float* dgu_s, uint8_t* dgu_qT, float* dgu_sT,
                        uint8_t* h_qT, float* h_sT, float* dgu_f32, float* h_f32,
                        int32_t flags, hipStream_t stream);

/* ---- combine [EP] ------------------------------------------------------- */

/* Weighted combine (the local half of the per-layer combine):
 *     y[t, :] = bf16( sum over local slots j, ascending, of w[t, j] * y_perm[pair_row[t, j], :] )
 * summed in fp32; tokens with no local pair get +0.  w == NULL uses weights of 1
 * (the unpermute-sum of the input gradient).
 *   y_perm [row_cap, d] bf16, pair_row [T, k], w [T, k] fp32, y [T, d] bf16.  */
int moe_unpermute_combine(const uint16_t* y_perm, const int32_t* pair_row, const float* w,
                          int64_t T, int32_t k, int32_t d, int64_t row_cap, uint16_t* y,
                          hipStream_t stream);

/* Combine backward: for every local pair (t, j) held by row r = pair_row[t, j]:
 *     dY[r, :]     = fp32(w[t, j] * dy[t, :])  -> 1x128 e4m3 (if dyq != NULL):
 *                    dyq [row_cap, d] u8, dyq_s [d/128, row_cap] fp32 (K-block-major)
 *     d_gate[t, j] = sum_n dy[t, n] * y_perm[r, n]   (fp32; 0 for non-local slots)
 *   dy [T, d] bf16, y_perm [row_cap, d] bf16 (the forward's expert outputs),
 *   pair_row [T, k], w [T, k] fp32, d_gate [T, k] fp32.
 * The 128x1 transposed copy of dY for wgrad comes from moe_quant_fp8_rows_t.
 * flags: 0, or MOE_SCALE_POW2 for power-of-two dyq_s scales.                  */
int moe_combine_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* pair_row,
                         const float* w, int64_t T, int32_t k, int32_t d, int64_t row_cap,
                         uint8_t* dyq, float* dyq_s, float* d_gate, int32_t flags,
                         hipStream_t stream);

/* Combine backward on the expert-grouped rows ("RL at 1T scale", section "FP8
 * Training": each backward GEMM operand quantised along its contraction axis):
 * one pass over dy and y_perm gives, for every real row r of the grouped layout
 * (pair p = row_pair[r] >= 0, token t = p / k, slot j = p % k):
 *     dY[r, :] = fp32(w[p] * dy[t, :])
 *       -> 1x128 e4m3:  dyq [row_cap, d] u8, dyq_s [d/128, row_cap] fp32
 *                       (as moe_combine_backward; padding rows not written)
 *       -> 128x1 e4m3 along rows, block-transposed: dyqT [row_cap/128, d, 128] u8,
 *                       dyqT_s [row_cap/128, d] fp32 (as moe_quant_fp8_rows_t
 *                       with w; padding rows count as 0)
 *     gate_part [row_cap, MOE_GATE_PARTS] fp32: entry (r, g) is the fp32 partial
 *       sum of dy[t, n] * y_perm[r, n] over the columns n of group g (groups of
 *       whole 128-column chunks; how many depends on d only); written for real
 *       rows and the groups d has, read back by moe_gate_backward_parts.
 * Rows at and past offsets[L] are not touched.  dy [T, d] bf16, y_perm
 * [row_cap, d] bf16 (the forward's expert outputs), w [T*k] fp32, row_pair
 * [row_cap], offsets [L+1] as written by moe_permute; d % 128 == 0,
 * row_cap % 128 == 0, row_cap * d and T * d below 2^31 (MOE_ERR_SHAPE).
 * flags: 0, or MOE_SCALE_POW2 for power-of-two scales on both copies.        */
#define MOE_GATE_PARTS 16
int moe_combine_backward_rows(const uint16_t* dy, const uint16_t* y_perm, const float* w,
                              const int32_t* row_pair, const int32_t* offsets, int64_t T,
                              int32_t L, int64_t row_cap, int32_t k, int32_t d, uint8_t* dyq, float* dyq_s,
                              uint8_t* dyqT, float* dyqT_s, float* gate_part, int32_t flags,
                              hipStream_t stream);

/* Backward of the softmax over the selected logits (complete when every expert
 * is local; under expert parallelism d_gate must first be summed over GPUs):
 *     d_logits[t, ids[t, j]] += w[t, j] * (d_gate[t, j] - sum_j' w[t, j'] d_gate[t, j'])
 * and 0 at unselected experts.  d_logits [T, E] fp32.                          */
int moe_gate_backward(const float* d_gate, const float* w, const int32_t* ids, int64_t T,
                      int32_t k, int32_t E, float* d_logits, hipStream_t stream);

/* The same from the partials of moe_combine_backward_rows: first
 *     d_gate[t, j] = sum over the groups g of gate_part[pair_row[t, j], g]
 * (summed in a fixed order; 0 for non-local slots), written to d_gate [T, k],
 * then d_logits as moe_gate_backward.  d is the feature width the partials
 * were taken over; pair_row [T, k] as written by moe_permute.                  */
int moe_gate_backward_parts(const float* gate_part, const int32_t* pair_row, int64_t row_cap,
                            int32_t d, const float* w, const int32_t* ids, int64_t T, int32_t k,
                            int32_t E, float* d_gate, float* d_logits, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
