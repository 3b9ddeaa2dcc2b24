// Combine on one GPU's share of experts ("RL at 1T scale", sections "Wide
// Expert Parallelism" and "Expert Parallel": per-layer combine after the
// experts) and its backward.
#include "common.hpp"

namespace moe {

constexpr int CMAXK = 16;
constexpr int CBLOCK = 128;

// One block per token; each thread owns up to CPT 8-element chunks of the
// output row (chunks t, t + CBLOCK, ...).  Local slots are summed in ascending
// order in fp32.  For each local slot (a uniform branch) the thread's chunk
// loads are all issued before the first is used, so a token costs about one
// memory latency per local slot rather than one per chunk and slot.
constexpr int CPT = 8;
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
    for (int c0 = 0; c0 < nchunk; c0 += CBLOCK * CPT) {
        float acc[CPT][8];
#pragma unroll
        for (int q = 0; q < CPT; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
#pragma unroll
        for (int j = 0; j < CMAXK; ++j) {
            if (rows[j] < 0) continue;
            const uint16_t* src = y_perm + (int64_t)rows[j] * d;
            uint4 v[CPT];
#pragma unroll
            for (int q = 0; q < CPT; ++q) {
                const int c = c0 + q * CBLOCK + threadIdx.x;
                if (c < nchunk) v[q] = *reinterpret_cast<const uint4*>(src + c * 8);
            }
            const float wj = ws[j];
#pragma unroll
            for (int q = 0; q < CPT; ++q) {
                acc[q][0] = fmaf(wj, bf16_lo(v[q].x), acc[q][0]);
                acc[q][1] = fmaf(wj, bf16_hi(v[q].x), acc[q][1]);
                acc[q][2] = fmaf(wj, bf16_lo(v[q].y), acc[q][2]);
                acc[q][3] = fmaf(wj, bf16_hi(v[q].y), acc[q][3]);
                acc[q][4] = fmaf(wj, bf16_lo(v[q].z), acc[q][4]);
                acc[q][5] = fmaf(wj, bf16_hi(v[q].z), acc[q][5]);
                acc[q][6] = fmaf(wj, bf16_lo(v[q].w), acc[q][6]);
                acc[q][7] = fmaf(wj, bf16_hi(v[q].w), acc[q][7]);
            }
        }
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int c = c0 + q * CBLOCK + threadIdx.x;
            if (c >= nchunk) continue;
            uint4 o;
            o.x = cvt_bf16x2(acc[q][0], acc[q][1]);
            o.y = cvt_bf16x2(acc[q][2], acc[q][3]);
            o.z = cvt_bf16x2(acc[q][4], acc[q][5]);
            o.w = cvt_bf16x2(acc[q][6], acc[q][7]);
            *reinterpret_cast<uint4*>(y + t * d + c * 8) = o;
        }
    }
}

// One block per token.  Work unit: one 128-wide tile, 16 lanes x 8 values; the
// 8 lane groups take tiles g, g + 8, ..., TPG at a time.  For every local slot
// j: dY = fp32(w_j * dy) quantised 1x128 (the tile amax of the rounded
// products is fp32(|w_j| * amax|dy|) because rounding is monotonic), and the
// partial dot <dy, Y_r> for d_gate.  Per local slot (a uniform branch) the
// group's Y tile loads are issued together before any is used.  Two tiles per
// group and pass (four passes over d = 7168) keep the kernel at about 70
// registers, so enough tokens are in flight per CU to hide the row latency:
// measured at the training shape, 7 tiles per pass (one pass, 168 registers)
// 190 us, 4 tiles 166 us, 2 tiles 156 us.
constexpr int TPG = 2;
template <bool P2>
__global__ __launch_bounds__(CBLOCK) void combine_bwd_kernel(const uint16_t* __restrict__ dy,
                                                             const uint16_t* __restrict__ y_perm,
                                                             const int32_t* __restrict__ pair_row,
                                                             const float* __restrict__ w, int k, int d,
                                                             uint8_t* __restrict__ dyq, float* __restrict__ dyq_s,
                                                             float* __restrict__ d_gate, int64_t row_cap) {
    __shared__ float part[CBLOCK / 64][CMAXK];
    __shared__ int slot_row[CMAXK];
    __shared__ float slot_w[CMAXK];
    const int64_t t = blockIdx.x;
    const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;  // 8 groups of 16 lanes
    const int wave = threadIdx.x >> 6;
    const int ntile = d >> 7;
    // the token's slots (rows and weights) are staged in LDS once, while the
    // dy row loads: no slot then waits on a global load of its own row index
    if ((int)threadIdx.x < k) {
        slot_row[threadIdx.x] = pair_row[t * k + threadIdx.x];
        slot_w[threadIdx.x] = w[t * k + threadIdx.x];
    }
    bool staged = false;
    for (int t0 = 0; t0 < ntile; t0 += (CBLOCK / 16) * TPG) {
        float v[TPG][8], am[TPG];
#pragma unroll
        for (int q = 0; q < TPG; ++q) {
            const int tile = t0 + q * (CBLOCK / 16) + grp;
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (tile < ntile) raw = *reinterpret_cast<const uint4*>(dy + t * d + (int64_t)tile * 128 + sub * 8);
            v[q][0] = bf16_lo(raw.x); v[q][1] = bf16_hi(raw.x);
            v[q][2] = bf16_lo(raw.y); v[q][3] = bf16_hi(raw.y);
            v[q][4] = bf16_lo(raw.z); v[q][5] = bf16_hi(raw.z);
            v[q][6] = bf16_lo(raw.w); v[q][7] = bf16_hi(raw.w);
        }
#pragma unroll
        for (int q = 0; q < TPG; ++q) {
            float m = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[q][i]));
            am[q] = group_max<16>(m);
        }
        if (!staged) {
            __syncthreads();
            staged = true;
        }
        // one body for all slots (kept rolled: the quantiser makes it long);
        // a slot that is not local costs a skipped branch only
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            const int64_t r = slot_row[j];  // uniform
            if (r < 0) continue;
            float dot = 0.f;
            {
                const float wj = slot_w[j];
                uint4 ys[TPG];
#pragma unroll
                for (int q = 0; q < TPG; ++q) {
                    const int tile = t0 + q * (CBLOCK / 16) + grp;
                    if (tile < ntile)
                        ys[q] = *reinterpret_cast<const uint4*>(y_perm + r * d + (int64_t)tile * 128 + sub * 8);
                }
#pragma unroll
                for (int q = 0; q < TPG; ++q) {
                    const int tile = t0 + q * (CBLOCK / 16) + grp;
                    if (tile >= ntile) continue;
                    const int64_t col = (int64_t)tile * 128 + sub * 8;
                    const uint4 yr = ys[q];
                    dot = fmaf(v[q][0], bf16_lo(yr.x), dot);
                    dot = fmaf(v[q][1], bf16_hi(yr.x), dot);
                    dot = fmaf(v[q][2], bf16_lo(yr.y), dot);
                    dot = fmaf(v[q][3], bf16_hi(yr.y), dot);
                    dot = fmaf(v[q][4], bf16_lo(yr.z), dot);
                    dot = fmaf(v[q][5], bf16_hi(yr.z), dot);
                    dot = fmaf(v[q][6], bf16_lo(yr.w), dot);
                    dot = fmaf(v[q][7], bf16_hi(yr.w), dot);
                    if (dyq) {
                        const TileScale ts = tile_scale_t<P2>(fabsf(wj) * am[q]);
                        uint2 o;
                        o.x = cvt_e4m3x4((wj * v[q][0]) * ts.inv, (wj * v[q][1]) * ts.inv, (wj * v[q][2]) * ts.inv,
                                         (wj * v[q][3]) * ts.inv);
                        o.y = cvt_e4m3x4((wj * v[q][4]) * ts.inv, (wj * v[q][5]) * ts.inv, (wj * v[q][6]) * ts.inv,
                                         (wj * v[q][7]) * ts.inv);
                        *reinterpret_cast<uint2*>(dyq + r * d + col) = o;
                        if (sub == 0) dyq_s[tile * row_cap + r] = ts.s;  // K-block-major scales
                    }
                }
            }
            // this pass's partial of <dy, Y_r>, summed over the block's lanes
            const float s = group_sum<64>(dot);
            if ((threadIdx.x & 63) == 0) part[wave][j] = (t0 == 0 ? 0.f : part[wave][j]) + s;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < k) {
        const int j = threadIdx.x;
        float s = 0.f;
        if (slot_row[j] >= 0)
            for (int wv = 0; wv < CBLOCK / 64; ++wv) s += part[wv][j];
        d_gate[t * k + j] = s;
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
                                    float* dyq_s, float* d_gate, int32_t flags, hipStream_t stream) {
    MOE_REQUIRE(flags == 0 || flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED, "combine_backward: unknown flags 0x%x", flags);
    MOE_REQUIRE(T >= 0 && T <= 0x7FFFFFFF && k >= 1 && k <= CMAXK, MOE_ERR_SHAPE, "combine_backward: bad T/k");
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "combine_backward: d=%d must be a multiple of 128", d);
    MOE_REQUIRE(row_cap >= 0, MOE_ERR_SHAPE, "combine_backward: bad row_cap");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(dy && y_perm && pair_row && w && d_gate, MOE_ERR_NULL, "combine_backward: NULL argument");
    MOE_REQUIRE(!dyq == !dyq_s, MOE_ERR_NULL, "combine_backward: dyq and dyq_s go together");
    auto go = [&](auto kern) {
        kern<<<dim3((unsigned)T), dim3(CBLOCK), 0, stream>>>(dy, y_perm, pair_row, w, k, d, dyq, dyq_s, d_gate, row_cap);
    };
    flags ? go(combine_bwd_kernel<true>) : go(combine_bwd_kernel<false>);
    MOE_LAUNCH_CHECK("combine_bwd_kernel");
    return MOE_OK;
}
