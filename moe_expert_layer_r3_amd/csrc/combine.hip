// Combine on one GPU's share of experts ("RL at 1T scale", sections "Wide
// Expert Parallelism" and "Expert Parallel": per-layer combine after the
// experts) and its backward.
#include "common.hpp"
#include "gate_parts.hpp"

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


// Rows of the expert-grouped layout gathered from a [T, d] source (row r holds
// pair row_pair[r], token row_pair[r] / k), scaled by w[pair] if given, and
// quantised twice from one read: 1x128 along the features (row-major) and
// 128x1 along the rows (block-transposed).  GATE: the combine backward, with
// dy as the source, w required, and the partial dots <dy_t, Y_r> of the gate
// gradient taken on the way.
// Block (column group g, row block b of 128 rows), 512 threads; the group is
// `cpb` 128-wide column chunks, taken one after the other.  Thread (wave wv,
// lane l) owns rows 4*rq .. 4*rq + 3 of the block, rq = 4*wv + l/16, and
// columns 8*cg .. 8*cg + 7 of the chunk, cg = l % 16.  Per chunk:
//   * the 4 source rows it needs are gathered (and, GATE, the 4 rows of
//     y_perm read), all loads issued together and those of the next chunk
//     issued before this chunk is quantised; GATE: <dy_t, Y_r> over the
//     chunk's 128 columns is added to the row's partial (fp32: 8-term chains,
//     then the 16 lanes of the row);
//   * v = fp32(w * src): a row's 1x128 tile is the 16 lanes of the row
//     (maximum over 8 values, then over those lanes), stored as 8-byte words
//     of one 128-byte run; padding rows are not written;
//   * a column's 128x1 tile is the thread's 4 rows, the wave's 4 row quads
//     (lanes 16 apart) and the 8 waves through LDS; its codes go through a
//     transposed LDS tile to 16-byte stores of 128-byte columns (padding rows
//     count as 0).
// GATE: the row's partial over the group's columns is written to
// gate_part[r * MOE_GATE_PARTS + g]; moe_gate_backward_parts sums the groups.
constexpr int CBR_THREADS = 512;
template <bool P2, bool GATE>
__global__ __launch_bounds__(CBR_THREADS) void rows_quant2_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y_perm, const float* __restrict__ w,
    const int32_t* __restrict__ row_pair, const int32_t* __restrict__ offsets, int L, int64_t row_cap, int k, int d,
    int cpb, uint8_t* __restrict__ dyq, float* __restrict__ dyq_s, uint8_t* __restrict__ dyqT,
    float* __restrict__ dyqT_s, float* __restrict__ gate_part) {
    __shared__ __attribute__((aligned(16))) float cmax[CBR_THREADS / 64][128];
    __shared__ __attribute__((aligned(16))) float cinv[128];
    __shared__ __attribute__((aligned(16))) uint8_t tile_t[128][128 + 8];
    const int64_t b = blockIdx.y;
    const int grp = blockIdx.x;
    int64_t total = offsets[L];
    if (total > row_cap) total = row_cap;
    if (b * 128 >= total) return;  // whole block leaves together
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = wave * 4 + (lane >> 4);
    const int c8 = cg * 8;
    const int nchunk = d >> 7;
    // element offsets fit 32 bits (checked on the host: T*d and row_cap*d < 2^31)
    const uint32_t r0 = (uint32_t)b * 128 + rq * 4;  // the thread's first row
    const int4 pa = *reinterpret_cast<const int4*>(row_pair + r0);
    const int p[4] = {pa.x, pa.y, pa.z, pa.w};
    float wp[4];
    uint32_t tok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        wp[j] = p[j] >= 0 ? (GATE || w ? w[p[j]] : 1.f) : 0.f;
        tok[j] = p[j] >= 0 ? (uint32_t)(p[j] / k) * (uint32_t)d : 0u;
    }
    const uint32_t row0 = r0 * (uint32_t)d;
    float dot[4] = {0.f, 0.f, 0.f, 0.f};

    // the next chunk's rows are loaded while the current one is quantised
    uint4 rd[4], ry[4];
    auto load = [&](int cc) {
        const uint32_t col = (uint32_t)cc * 128 + c8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rd[j] = make_uint4(0, 0, 0, 0);
            ry[j] = make_uint4(0, 0, 0, 0);
            if (p[j] >= 0) {
                rd[j] = *reinterpret_cast<const uint4*>(dy + (tok[j] + col));
                if constexpr (GATE) ry[j] = *reinterpret_cast<const uint4*>(y_perm + (row0 + (uint32_t)j * d + col));
            }
        }
    };
    const int cc_end = min(nchunk, (grp + 1) * cpb);
    load(grp * cpb);
#pragma unroll 1
    for (int cc = grp * cpb; cc < cc_end; ++cc) {
        const uint32_t col = (uint32_t)cc * 128 + c8;
        float v[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j][0] = bf16_lo(rd[j].x); v[j][1] = bf16_hi(rd[j].x);
            v[j][2] = bf16_lo(rd[j].y); v[j][3] = bf16_hi(rd[j].y);
            v[j][4] = bf16_lo(rd[j].z); v[j][5] = bf16_hi(rd[j].z);
            v[j][6] = bf16_lo(rd[j].w); v[j][7] = bf16_hi(rd[j].w);
            if constexpr (GATE) {
                float s = v[j][0] * bf16_lo(ry[j].x);
                s = fmaf(v[j][1], bf16_hi(ry[j].x), s);
                s = fmaf(v[j][2], bf16_lo(ry[j].y), s);
                s = fmaf(v[j][3], bf16_hi(ry[j].y), s);
                s = fmaf(v[j][4], bf16_lo(ry[j].z), s);
                s = fmaf(v[j][5], bf16_hi(ry[j].z), s);
                s = fmaf(v[j][6], bf16_lo(ry[j].w), s);
                s = fmaf(v[j][7], bf16_hi(ry[j].w), s);
                dot[j] += s;
            }
        }
        if (cc + 1 < cc_end) load(cc + 1);
        // dY = fp32(w * dy); maxima of the rows (1x128) and of the columns (128x1)
        float am[8], rm[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) am[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rm[j] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[j][i] = wp[j] * v[j][i];
                const float a = fabsf(v[j][i]);
                am[i] = fmaxf(am[i], a);
                rm[j] = fmaxf(rm[j], a);
            }
        }
        // 1x128 tiles of the thread's rows: lane cg computes the scale of row
        // cg % 4 of its quad and the quad's lanes read the four back
#pragma unroll
        for (int j = 0; j < 4; ++j) rm[j] = group_max<16>(rm[j]);
        const TileScale ts_own = tile_scale_t<P2>(cg & 2 ? (cg & 1 ? rm[3] : rm[2]) : (cg & 1 ? rm[1] : rm[0]));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float inv = __shfl(ts_own.inv, (lane & 48) + j);
            if (p[j] >= 0) {
                uint2 o;
                o.x = cvt_e4m3x4(v[j][0] * inv, v[j][1] * inv, v[j][2] * inv, v[j][3] * inv);
                o.y = cvt_e4m3x4(v[j][4] * inv, v[j][5] * inv, v[j][6] * inv, v[j][7] * inv);
                *reinterpret_cast<uint2*>(dyq + (row0 + (uint32_t)j * d + col)) = o;
            }
        }
        if (cg < 4 && p[cg & 3] >= 0) dyq_s[(uint32_t)cc * (uint32_t)row_cap + r0 + cg] = ts_own.s;  // K-block-major
        // 128x1 tiles of the chunk's columns: maxima over the thread's rows, the
        // wave's row quads and (through LDS) the waves; thread c < 128 forms
        // column c's scale
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            am[i] = fmaxf(am[i], __shfl_xor(am[i], 16));
            am[i] = fmaxf(am[i], __shfl_xor(am[i], 32));
        }
        if (lane < 16) {
            *reinterpret_cast<float4*>(&cmax[wave][c8]) = make_float4(am[0], am[1], am[2], am[3]);
            *reinterpret_cast<float4*>(&cmax[wave][c8 + 4]) = make_float4(am[4], am[5], am[6], am[7]);
        }
        __syncthreads();
        if (tid < 128) {
            float m = cmax[0][tid];
#pragma unroll
            for (int wv = 1; wv < CBR_THREADS / 64; ++wv) m = fmaxf(m, cmax[wv][tid]);
            const TileScale ts = tile_scale_t<P2>(m);
            cinv[tid] = ts.inv;
            dyqT_s[(uint32_t)b * d + (uint32_t)cc * 128 + tid] = ts.s;  // token-block-major
        }
        __syncthreads();
        const float4 i0 = *reinterpret_cast<const float4*>(&cinv[c8]);
        const float4 i1 = *reinterpret_cast<const float4*>(&cinv[c8 + 4]);
        const float ci[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint32_t*>(&tile_t[c8 + i][rq * 4]) =
                cvt_e4m3x4(v[0][i] * ci[i], v[1][i] * ci[i], v[2][i] * ci[i], v[3][i] * ci[i]);
        __syncthreads();
        for (int idx = tid; idx < 128 * 8; idx += CBR_THREADS) {
            const int c = idx >> 3, part = (idx & 7) * 16;
            const uint4 val = *reinterpret_cast<const uint4*>(&tile_t[c][part]);
            *reinterpret_cast<uint4*>(dyqT + ((((uint32_t)b * d + (uint32_t)cc * 128 + c) << 7) + part)) = val;
        }
    }
    if constexpr (!GATE) return;
    // the rows' partials over this group's columns; lane cg == j writes row j's
    float own = 0.f;
    bool real_own = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float s = group_sum<16>(dot[j]);
        if (cg == j) {
            own = s;
            real_own = p[j] >= 0;
        }
    }
    if (real_own) gate_part[(r0 + cg) * MOE_GATE_PARTS + grp] = own;
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

extern "C" int moe_combine_backward_rows(const uint16_t* dy, const uint16_t* y_perm, const float* w,
                                         const int32_t* row_pair, const int32_t* offsets, int64_t T, int32_t L,
                                         int64_t row_cap,
                                         int32_t k, int32_t d, uint8_t* dyq, float* dyq_s, uint8_t* dyqT,
                                         float* dyqT_s, float* gate_part, int32_t flags, hipStream_t stream) {
    MOE_REQUIRE(flags == 0 || flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED,
                "combine_backward_rows: unknown flags 0x%x", flags);
    MOE_REQUIRE(L >= 1 && L <= 1024 && k >= 1 && k <= CMAXK, MOE_ERR_SHAPE, "combine_backward_rows: bad L/k");
    MOE_REQUIRE(row_cap >= 0 && row_cap % 128 == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "combine_backward_rows: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "combine_backward_rows: d=%d must be a multiple of 128", d);
    if (row_cap == 0) return MOE_OK;
    MOE_REQUIRE(dy && y_perm && w && row_pair && offsets && dyq && dyq_s && dyqT && dyqT_s && gate_part, MOE_ERR_NULL,
                "combine_backward_rows: NULL argument");
    MOE_REQUIRE(row_cap / 128 <= 65535, MOE_ERR_SHAPE, "combine_backward_rows: row_cap too large");
    // 32-bit element offsets in the kernel: the dyqT byte offsets are the largest (row_cap * d)
    MOE_REQUIRE(row_cap * d < ((int64_t)1 << 31) && T >= 0 && T * d < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "combine_backward_rows: row_cap * d and T * d must stay below 2^31");
    const int cpb = gate_chunks_per_group(d);
    dim3 grid((unsigned)gate_groups(d), (unsigned)(row_cap / 128));
    auto go = [&](auto kern) {
        kern<<<grid, CBR_THREADS, 0, stream>>>(dy, y_perm, w, row_pair, offsets, L, row_cap, k, d, cpb, dyq, dyq_s, dyqT,
                                       dyqT_s, gate_part);
    };
    flags ? go(rows_quant2_kernel<true, true>) : go(rows_quant2_kernel<false, true>);
    MOE_LAUNCH_CHECK("rows_quant2_kernel");
    return MOE_OK;
}

extern "C" int moe_quant_fp8_rows_both(const uint16_t* src, const float* w, const int32_t* row_pair,
                                       const int32_t* offsets, int64_t T, int32_t L, int64_t row_cap, int32_t k,
                                       int32_t cols, uint8_t* q, float* q_s, uint8_t* qT, float* qT_s,
                                       int32_t flags, hipStream_t stream) {
    MOE_REQUIRE(flags == 0 || flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED, "quant_fp8_rows_both: unknown flags 0x%x",
                flags);
    MOE_REQUIRE(L >= 1 && L <= 1024 && k >= 1 && k <= CMAXK, MOE_ERR_SHAPE, "quant_fp8_rows_both: bad L/k");
    MOE_REQUIRE(row_cap >= 0 && row_cap % 128 == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "quant_fp8_rows_both: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_SHAPE, "quant_fp8_rows_both: cols=%d must be a multiple of 128",
                cols);
    if (row_cap == 0) return MOE_OK;
    MOE_REQUIRE(src && row_pair && offsets && q && q_s && qT && qT_s, MOE_ERR_NULL,
                "quant_fp8_rows_both: NULL argument");
    MOE_REQUIRE(row_cap / 128 <= 65535, MOE_ERR_SHAPE, "quant_fp8_rows_both: row_cap too large");
    MOE_REQUIRE(row_cap * cols < ((int64_t)1 << 31) && T >= 0 && T * cols < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "quant_fp8_rows_both: row_cap * cols and T * cols must stay below 2^31");
    const int cpb = gate_chunks_per_group(cols);
    dim3 grid((unsigned)gate_groups(cols), (unsigned)(row_cap / 128));
    auto go = [&](auto kern) {
        kern<<<grid, CBR_THREADS, 0, stream>>>(src, nullptr, w, row_pair, offsets, L, row_cap, k, cols, cpb, q, q_s,
                                               qT, qT_s, nullptr);
    };
    flags ? go(rows_quant2_kernel<true, false>) : go(rows_quant2_kernel<false, false>);
    MOE_LAUNCH_CHECK("rows_quant2_kernel");
    return MOE_OK;
}
