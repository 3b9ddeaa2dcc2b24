// Thin last m-tiles of the SwiGLU grouped GEMM, split along K.
//
// The 256-column SwiGLU product runs 288-row m-tiles, one persistent
// workgroup per tile at a time.  An expert whose rows leave at most THIN_ROWS
// rows for its last m-tile (one with 289-320 rows, say) still gives that tile
// a whole K loop: one workgroup streams the expert's full weight tile for a
// few rows, one K step after another at memory latency, and when the tile
// count just passes a multiple of the workgroup count those tiles form a last
// round of their own (measured at the ep8 shape: 528 tiles on 256 workgroups,
// 419 us against 308 us for 512).  With MOE_GEMM_THIN_SPLIT the main product
// leaves those rows out, and two small launches compute them: every (thin
// expert, n-tile, run of THIN_KB K blocks) is one work item writing an fp32
// partial to the caller's workspace, and a second launch sums the partials in
// K order and applies the same SwiGLU epilogue.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int THIN_WBM = 288;   // rows of the SwiGLU product's m-tiles
constexpr int THIN_ROWS = 32;   // a last m-tile of at most this many rows is thin
constexpr int THIN_KB = 4;      // K blocks (of 128) per work item

// K runs per (expert, n-tile)
__host__ __device__ inline int thin_splits(int K) { return (K / 128 + THIN_KB - 1) / THIN_KB; }

// rows of the expert's segment that the product covers, given its count and
// segment bounds (both clipped to row_cap)
__device__ __forceinline__ int64_t thin_seg_rows(const int32_t* counts, const int32_t* offsets, int e,
                                                 int64_t row_cap) {
    int64_t lo = offsets[e], hi = offsets[e + 1];
    if (lo > row_cap) lo = row_cap;
    if (hi > row_cap) hi = row_cap;
    int64_t rows = counts[e];
    if (rows > hi - lo) rows = hi - lo;
    return rows > 0 ? rows : 0;
}

// rows of the expert's last m-tile when that tile is thin, else 0
__device__ __forceinline__ int thin_rows_of(int64_t rows) {
    if (rows <= 0) return 0;
    const int64_t m = (rows + THIN_WBM - 1) / THIN_WBM;
    const int64_t last = rows - (int64_t)THIN_WBM * (m - 1);
    return last <= THIN_ROWS ? (int)last : 0;
}

// With m_tiles m-tiles over all experts, thin of them thin, NT n-tiles and G
// persistent workgroups: the thin tiles are split off only when they add a
// round of tiles (ceil(tiles / G) drops without them); otherwise they ride in
// the main product's rounds at no extra cost.
__host__ __device__ inline bool thin_split_active(int m_tiles, int thin, int NT, int G) {
    if (thin <= 0 || G <= 0) return false;
    const int64_t all = (int64_t)m_tiles * NT, rest = (int64_t)(m_tiles - thin) * NT;
    return (all + G - 1) / G > (rest + G - 1) / G;
}

}  // namespace moe

// bytes of the fp32 partials for every expert of a product with N = 2f, K
size_t moe_thin_workspace_bytes(int32_t L, int32_t N, int32_t K);
// the K-split launches for the thin last m-tiles (after the main product, on
// the same stream); ws holds moe_thin_workspace_bytes(L, N, K)
int moe_thin_launch(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s, const int32_t* counts,
                    const int32_t* offsets, int32_t L, int64_t row_cap, int32_t N, int32_t K, int32_t epilogue,
                    bool p2, float* ws, void* out, float* out_s, void* out2, hipStream_t stream);
