// Combine on one GPU's share of experts ("RL at 1T scale", sections "Wide
// Expert Parallelism" and "Expert Parallel": per-layer combine after the
// experts) and its backward.
#include "common.hpp"

namespace moe {

constexpr int CMAXK = 16;
constexpr int CBLOCK = 128;

// One block per token; each thread owns 8-element chunks of the output row.
// Local slots are summed in ascending order in fp32.
__global__ __launch_bounds__(CBLOCK) void combine_kernel(const uint16_t* __restrict__ y_perm,
                                                         const int32_t* __restrict__ pair_row,
                                                         const float* __restrict__ w, int k, int d,
                                                         uint16_t* __restrict__ y) {
    const int64_t t = blockIdx.x;
    int rows[CMAXK];
    float ws[CMAXK];
#pragma unroll
    for (int j = 0; j < CMAXK; ++j) {
        rows[j] = j < k ? pair_row[t * k + j] : -1;
        ws[j] = (j < k && w) ? w[t * k + j] : 1.f;
    }
    const int nchunk = d >> 3;
    for (int c = threadIdx.x; c < nchunk; c += CBLOCK) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < CMAXK; ++j) {
            if (rows[j] >= 0) {
                const uint4 v = *reinterpret_cast<const uint4*>(y_perm + (int64_t)rows[j] * d + c * 8);
                const float wj = ws[j];
                acc[0] = fmaf(wj, bf16_lo(v.x), acc[0]);
                acc[1] = fmaf(wj, bf16_hi(v.x), acc[1]);
                acc[2] = fmaf(wj, bf16_lo(v.y), acc[2]);
                acc[3] = fmaf(wj, bf16_hi(v.y), acc[3]);
                acc[4] = fmaf(wj, bf16_lo(v.z), acc[4]);
                acc[5] = fmaf(wj, bf16_hi(v.z), acc[5]);
                acc[6] = fmaf(wj, bf16_lo(v.w), acc[6]);
                acc[7] = fmaf(wj, bf16_hi(v.w), acc[7]);
            }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(y + t * d + c * 8) = o;
    }
}

// One block per token.  Work unit: one 128-wide tile, 16 lanes x 8 values.
// For every local slot j: dY = fp32(w_j * dy) quantised 1x128 (the tile amax of
// the rounded products is fp32(|w_j| * amax|dy|) because rounding is
// monotonic), and the partial dot <dy, Y_r> for d_gate.
__global__ __launch_bounds__(CBLOCK) void combine_bwd_kernel(const uint16_t* __restrict__ dy,
                                                             const uint16_t* __restrict__ y_perm,
                                                             const int32_t* __restrict__ pair_row,
                                                             const float* __restrict__ w, int k, int d,
                                                             uint8_t* __restrict__ dyq, float* __restrict__ dyq_s,
                                                             float* __restrict__ d_gate, int64_t row_cap) {
    __shared__ float part[CBLOCK / 64][CMAXK];
    const int64_t t = blockIdx.x;
    const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;  // 8 groups of 16 lanes
    const int ntile = d >> 7;
    int rows[CMAXK];
    float ws[CMAXK], dot[CMAXK];
#pragma unroll
    for (int j = 0; j < CMAXK; ++j) {
        rows[j] = j < k ? pair_row[t * k + j] : -1;
        ws[j] = j < k ? w[t * k + j] : 0.f;
        dot[j] = 0.f;
    }
    for (int tile = grp; tile < ntile; tile += CBLOCK / 16) {
        const int64_t col = (int64_t)tile * 128 + sub * 8;
        const uint4 raw = *reinterpret_cast<const uint4*>(dy + t * d + col);
        float v[8];
        v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
        v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
        v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
        v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
        am = group_max<16>(am);
#pragma unroll
        for (int j = 0; j < CMAXK; ++j) {
            if (rows[j] < 0) continue;
            const int64_t r = rows[j];
            const float wj = ws[j];
            const uint4 yr = *reinterpret_cast<const uint4*>(y_perm + r * d + col);
            dot[j] = fmaf(v[0], bf16_lo(yr.x), dot[j]);
            dot[j] = fmaf(v[1], bf16_hi(yr.x), dot[j]);
            dot[j] = fmaf(v[2], bf16_lo(yr.y), dot[j]);
            dot[j] = fmaf(v[3], bf16_hi(yr.y), dot[j]);
            dot[j] = fmaf(v[4], bf16_lo(yr.z), dot[j]);
            dot[j] = fmaf(v[5], bf16_hi(yr.z), dot[j]);
            dot[j] = fmaf(v[6], bf16_lo(yr.w), dot[j]);
            dot[j] = fmaf(v[7], bf16_hi(yr.w), dot[j]);
            if (dyq) {
                TileScale ts = tile_scale(fabsf(wj) * am);
                uint2 o;
                o.x = cvt_e4m3x4((wj * v[0]) * ts.inv, (wj * v[1]) * ts.inv, (wj * v[2]) * ts.inv,
                                 (wj * v[3]) * ts.inv);
                o.y = cvt_e4m3x4((wj * v[4]) * ts.inv, (wj * v[5]) * ts.inv, (wj * v[6]) * ts.inv,
                                 (wj * v[7]) * ts.inv);
                *reinterpret_cast<uint2*>(dyq + r * d + col) = o;
                if (sub == 0) dyq_s[tile * row_cap + r] = ts.s;  // K-block-major scales
            }
        }
    }
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < CMAXK; ++j) {
        float s = group_sum<64>(dot[j]);
        if ((threadIdx.x & 63) == 0) part[wave][j] = s;
    }
    __syncthreads();
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        float s = 0.f;
        for (int wv = 0; wv < CBLOCK / 64; ++wv) s += part[wv][j];
        d_gate[t * k + j] = pair_row[t * k + j] >= 0 ? s : 0.f;
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_unpermute_combine(const uint16_t* y_perm, const int32_t* pair_row, const float* w, int64_t T,
                                     int32_t k, int32_t d, int64_t row_cap, uint16_t* y, hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && T <= 0x7FFFFFFF && k >= 1 && k <= CMAXK, MOE_ERR_SHAPE, "combine: bad T/k");
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "combine: d=%d must be a multiple of 128", d);
    MOE_REQUIRE(row_cap >= 0, MOE_ERR_SHAPE, "combine: bad row_cap");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(pair_row && y && (row_cap == 0 || y_perm), MOE_ERR_NULL, "combine: NULL argument");
    combine_kernel<<<dim3((unsigned)T), dim3(CBLOCK), 0, stream>>>(y_perm, pair_row, w, k, d, y);
    MOE_LAUNCH_CHECK("combine_kernel");
    return MOE_OK;
}

extern "C" int moe_combine_backward(const uint16_t* dy, const uint16_t* y_perm, const int32_t* pair_row,
                                    const float* w, int64_t T, int32_t k, int32_t d, int64_t row_cap, uint8_t* dyq,
                                    float* dyq_s, float* d_gate, hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && T <= 0x7FFFFFFF && k >= 1 && k <= CMAXK, MOE_ERR_SHAPE, "combine_backward: bad T/k");
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "combine_backward: d=%d must be a multiple of 128", d);
    MOE_REQUIRE(row_cap >= 0, MOE_ERR_SHAPE, "combine_backward: bad row_cap");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(dy && y_perm && pair_row && w && d_gate, MOE_ERR_NULL, "combine_backward: NULL argument");
    MOE_REQUIRE(!dyq == !dyq_s, MOE_ERR_NULL, "combine_backward: dyq and dyq_s go together");
    combine_bwd_kernel<<<dim3((unsigned)T), dim3(CBLOCK), 0, stream>>>(dy, y_perm, pair_row, w, k, d, dyq, dyq_s,
                                                                       d_gate, row_cap);
    MOE_LAUNCH_CHECK("combine_bwd_kernel");
    return MOE_OK;
}
