// Block-scaled FP8 e4m3 quantisation ("RL at 1T scale", section "FP8 Training":
// DeepSeek-V3 style block scaling).  Per tile: a = max(max|v|, 2^-40),
// inv = 448/a, s = a/448 (fp32, correctly rounded), q = e4m3_rne_sat(fp32(v*inv)).
// With P2 the scale is the power of two s = 2^e, e the least integer with
// a <= 448 * 2^e (a UE8M0 code), and inv = 2^-e exactly.
#include "common.hpp"

namespace moe {

template <bool F32>
__device__ __forceinline__ void load8(const void* src, int64_t idx, float v[8]) {
    if (F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + idx);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + idx);
        v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x);
        v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
        v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z);
        v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
    }
}

// 1x128: a work item is one 128-wide tile of one row, 16 lanes x 8 values.
template <bool F32, bool P2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ src, int64_t nrows, int64_t cols,
                                                          int64_t ld, uint8_t* __restrict__ q,
                                                          float* __restrict__ s) {
    const int64_t ntile = cols >> 7;
    const int64_t item = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
    const int sub = threadIdx.x & 15;
    if (item >= nrows * ntile) return;  // whole 16-lane groups leave together
    const int64_t r = item / ntile, tile = item - r * ntile;
    const int64_t col = tile * 128 + sub * 8;
    float v[8];
    load8<F32>(src, r * ld + col, v);
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = group_max<16>(am);
    TileScale ts = tile_scale_t<P2>(am);
    uint2 out;
    out.x = cvt_e4m3x4(v[0] * ts.inv, v[1] * ts.inv, v[2] * ts.inv, v[3] * ts.inv);
    out.y = cvt_e4m3x4(v[4] * ts.inv, v[5] * ts.inv, v[6] * ts.inv, v[7] * ts.inv);
    *reinterpret_cast<uint2*>(q + r * cols + col) = out;
    if (sub == 0) s[r * ntile + tile] = ts.s;
}

// 128x128: one block of 256 threads per tile.  Thread (wave w, lane l) covers
// rows 8*rq .. 8*rq + 7 of the tile, rq = 4w + l/16, and columns 8*cg .. +7,
// cg = l % 16 (16 lanes read a row's 256 bytes).  The optional transposed copy
// goes through an LDS tile: a column's codes for the thread's 8 consecutive
// rows are one 8-byte word.
template <bool F32, bool P2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const void* __restrict__ src, int64_t rows,
                                                            int64_t cols, int64_t ld, uint8_t* __restrict__ q,
                                                            float* __restrict__ s, uint8_t* __restrict__ qT,
                                                            float* __restrict__ sT) {
    __shared__ float wmax[4];
    __shared__ __attribute__((aligned(16))) uint8_t tile_t[128][128 + 8];
    const int64_t rb_n = rows >> 7, cb_n = cols >> 7;
    const int64_t g = blockIdx.z;
    // tiles in row-major order, contiguous per XCD: the tiles one XCD runs side
    // by side cover whole rows of the source (adjacent 256-byte pieces of each
    // row) instead of every eighth piece
    const int64_t lin = xcd_tile((int64_t)blockIdx.y * cb_n + blockIdx.x, rb_n * cb_n);
    const int64_t rb = lin / cb_n, cb = lin - rb * cb_n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = wave * 4 + (lane >> 4);
    const int c8 = cg * 8;
    const int64_t gbase = g * rows * ld;
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = rb * 128 + rq * 8 + j;
        load8<F32>(src, gbase + r * ld + cb * 128 + c8, v[j]);
    }
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[j][i]));
    am = group_max<64>(am);
    if (lane == 0) wmax[wave] = am;
    __syncthreads();
    am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const TileScale ts = tile_scale_t<P2>(am);
    const int64_t qbase = g * rows * cols;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint2 out;
        out.x = cvt_e4m3x4(v[j][0] * ts.inv, v[j][1] * ts.inv, v[j][2] * ts.inv, v[j][3] * ts.inv);
        out.y = cvt_e4m3x4(v[j][4] * ts.inv, v[j][5] * ts.inv, v[j][6] * ts.inv, v[j][7] * ts.inv);
        // streaming store: the codes are not read again before they leave the caches
        __builtin_nontemporal_store(((uint64_t)out.y << 32) | out.x,
                                    reinterpret_cast<uint64_t*>(q + qbase + (rb * 128 + rq * 8 + j) * cols + cb * 128 + c8));
    }
    if (tid == 0) {
        s[(g * rb_n + rb) * cb_n + cb] = ts.s;
        if (sT) sT[(g * cb_n + cb) * rb_n + rb] = ts.s;
    }
    if (qT) {
        // column c8 + i, rows 8rq .. 8rq + 7 (the same rounding as above)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = cvt_e4m3x4(v[0][i] * ts.inv, v[1][i] * ts.inv, v[2][i] * ts.inv, v[3][i] * ts.inv);
            const uint32_t hi = cvt_e4m3x4(v[4][i] * ts.inv, v[5][i] * ts.inv, v[6][i] * ts.inv, v[7][i] * ts.inv);
            *reinterpret_cast<uint2*>(&tile_t[c8 + i][rq * 8]) = make_uint2(lo, hi);
        }
        __syncthreads();
        // qT[g][c][r]: 128 rows of the transposed tile, 16 bytes per thread per step
        for (int idx = tid; idx < 128 * 8; idx += 256) {
            const int c = idx >> 3, part = (idx & 7) * 16;
            const uint4 val = *reinterpret_cast<const uint4*>(&tile_t[c][part]);
            *reinterpret_cast<uint4*>(qT + qbase + (cb * 128 + c) * rows + rb * 128 + part) = val;
        }
    }
}

// 128x1 along rows of the expert-grouped layout with the row gather fused,
// block-transposed output.  Block (column chunk cc of 128, row block b of 128),
// 256 threads.  Thread (wave w, lane l) owns rows 8*rq .. 8*rq + 7 of the block,
// rq = 4w + l/16, and columns 8*cg .. 8*cg + 7, cg = l % 16:
//   * the 16 lanes of one row read its 256 contiguous bytes, and the thread's
//     8 row ids are one 32-byte load, all issued before any use;
//   * a column's maximum is the thread's 8 rows, then the wave's 4 row octets
//     (lanes 16 apart), then the 4 waves through a small LDS array;
//   * a column's codes for the thread's 8 consecutive rows are one 8-byte word
//     of the transposed LDS tile, which leaves as 16-byte stores of full
//     128-byte columns.
template <bool P2>
__global__ __launch_bounds__(256) void quant_rows_t_kernel(const uint16_t* __restrict__ src,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ row_pair,
                                                           const int32_t* __restrict__ offsets, int L,
                                                           int64_t row_cap, int k, int64_t cols,
                                                           uint8_t* __restrict__ qT, float* __restrict__ sT) {
    __shared__ __attribute__((aligned(16))) float cmax[4][128];
    __shared__ __attribute__((aligned(16))) uint8_t tile_t[128][128 + 8];
    const int64_t b = blockIdx.y, cc = blockIdx.x;
    int64_t total = offsets[L];
    if (total > row_cap) total = row_cap;
    if (b * 128 >= total) return;  // whole block leaves together
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = wave * 4 + (lane >> 4);
    const int c8 = cg * 8;
    const int4* rp = reinterpret_cast<const int4*>(row_pair + b * 128 + rq * 8);
    const int4 pa = rp[0], pb = rp[1];
    const int p[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    float wp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wp[j] = (w && p[j] >= 0) ? w[p[j]] : 1.f;
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (p[j] >= 0) {
            load8<false>(src, (int64_t)(p[j] / k) * cols + cc * 128 + c8, v[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
        }
    }
    float am[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) am[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (w) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[j][i] = wp[j] * v[j][i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) am[i] = fmaxf(am[i], fabsf(v[j][i]));
    }
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
    float inv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float m = fmaxf(fmaxf(cmax[0][c8 + i], cmax[1][c8 + i]), fmaxf(cmax[2][c8 + i], cmax[3][c8 + i]));
        const TileScale ts = tile_scale_t<P2>(m);
        inv[i] = ts.inv;
        if (wave == 0 && lane < 16) sT[b * cols + cc * 128 + c8 + i] = ts.s;  // token-block-major scales
    }
    // column c8 + i, rows 8rq .. 8rq + 7: bytes 0..7 of one word
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = inv[i];
        const uint32_t lo = cvt_e4m3x4(v[0][i] * x, v[1][i] * x, v[2][i] * x, v[3][i] * x);
        const uint32_t hi = cvt_e4m3x4(v[4][i] * x, v[5][i] * x, v[6][i] * x, v[7][i] * x);
        *reinterpret_cast<uint2*>(&tile_t[c8 + i][rq * 8]) = make_uint2(lo, hi);
    }
    __syncthreads();
    for (int idx = tid; idx < 128 * 8; idx += 256) {
        const int c = idx >> 3, part = (idx & 7) * 16;
        const uint4 val = *reinterpret_cast<const uint4*>(&tile_t[c][part]);
        *reinterpret_cast<uint4*>(qT + ((b * cols + cc * 128 + c) << 7) + part) = val;
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_quant_fp8(const void* src, int32_t src_type, int64_t groups, int64_t rows, int64_t cols,
                             int64_t ld, int32_t tile, uint8_t* q, float* scales, uint8_t* qT, float* scalesT,
                             hipStream_t stream) {
    MOE_REQUIRE(src_type == MOE_SRC_BF16 || src_type == MOE_SRC_F32, MOE_ERR_UNSUPPORTED,
                "quant_fp8: unknown src_type %d", src_type);
    const bool p2 = (tile & MOE_SCALE_POW2) != 0;
    tile &= ~MOE_SCALE_POW2;
    MOE_REQUIRE(tile == MOE_TILE_1x128 || tile == MOE_TILE_128x128, MOE_ERR_UNSUPPORTED,
                "quant_fp8: unknown tile %d", tile);
    MOE_REQUIRE(groups >= 0 && rows >= 0 && cols >= 0 && cols % 128 == 0, MOE_ERR_SHAPE,
                "quant_fp8: cols=%lld must be a multiple of 128", (long long)cols);
    MOE_REQUIRE(ld >= cols && ld % 8 == 0, MOE_ERR_SHAPE, "quant_fp8: ld=%lld must be >= cols and a multiple of 8",
                (long long)ld);
    MOE_REQUIRE(tile == MOE_TILE_1x128 || rows % 128 == 0, MOE_ERR_SHAPE,
                "quant_fp8: 128x128 tiles need rows %% 128 == 0 (rows=%lld)", (long long)rows);
    MOE_REQUIRE(tile == MOE_TILE_128x128 || (!qT && !scalesT), MOE_ERR_UNSUPPORTED,
                "quant_fp8: the transposed copy exists for 128x128 tiles only");
    MOE_REQUIRE(!qT == !scalesT, MOE_ERR_NULL, "quant_fp8: qT and scalesT go together");
    if (groups == 0 || rows == 0 || cols == 0) return MOE_OK;
    MOE_REQUIRE(src && q && scales, MOE_ERR_NULL, "quant_fp8: NULL src/q/scales");
    const bool f32 = src_type == MOE_SRC_F32;
    if (tile == MOE_TILE_1x128) {
        // groups of [rows, cols] with stride rows*ld are one [groups*rows, cols] matrix
        const int64_t nrows = groups * rows;
        const int64_t threads = nrows * (cols / 128) * 16;
        dim3 grid((unsigned)((threads + 255) / 256));
        auto go = [&](auto kern) { kern<<<grid, 256, 0, stream>>>(src, nrows, cols, ld, q, scales); };
        if (f32)
            p2 ? go(quant_1x128_kernel<true, true>) : go(quant_1x128_kernel<true, false>);
        else
            p2 ? go(quant_1x128_kernel<false, true>) : go(quant_1x128_kernel<false, false>);
        MOE_LAUNCH_CHECK("quant_1x128_kernel");
    } else {
        MOE_REQUIRE(rows / 128 <= 65535 && groups <= 65535, MOE_ERR_SHAPE, "quant_fp8: too many 128x128 tiles");
        dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128), (unsigned)groups);
        auto go = [&](auto kern) { kern<<<grid, 256, 0, stream>>>(src, rows, cols, ld, q, scales, qT, scalesT); };
        if (f32)
            p2 ? go(quant_128x128_kernel<true, true>) : go(quant_128x128_kernel<true, false>);
        else
            p2 ? go(quant_128x128_kernel<false, true>) : go(quant_128x128_kernel<false, false>);
        MOE_LAUNCH_CHECK("quant_128x128_kernel");
    }
    return MOE_OK;
}

extern "C" int moe_quant_fp8_rows_t(const uint16_t* src, const float* w, const int32_t* row_pair,
                                    const int32_t* offsets, int32_t L, int64_t row_cap, int32_t k, int64_t cols,
                                    uint8_t* qT, float* sT, int32_t flags, hipStream_t stream) {
    MOE_REQUIRE(flags == 0 || flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED, "quant_fp8_rows_t: unknown flags 0x%x", flags);
    MOE_REQUIRE(L >= 1 && L <= 1024 && k >= 1 && k <= 16, MOE_ERR_SHAPE, "quant_fp8_rows_t: bad L/k");
    MOE_REQUIRE(row_cap >= 0 && row_cap % 128 == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "quant_fp8_rows_t: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_SHAPE, "quant_fp8_rows_t: cols=%lld must be a multiple of 128",
                (long long)cols);
    if (row_cap == 0) return MOE_OK;
    MOE_REQUIRE(src && row_pair && offsets && qT && sT, MOE_ERR_NULL, "quant_fp8_rows_t: NULL argument");
    MOE_REQUIRE(row_cap / 128 <= 65535, MOE_ERR_SHAPE, "quant_fp8_rows_t: row_cap too large");
    dim3 grid((unsigned)(cols / 128), (unsigned)(row_cap / 128));
    auto go = [&](auto kern) { kern<<<grid, 256, 0, stream>>>(src, w, row_pair, offsets, L, row_cap, k, cols, qT, sT); };
    flags ? go(quant_rows_t_kernel<true>) : go(quant_rows_t_kernel<false>);
    MOE_LAUNCH_CHECK("quant_rows_t_kernel");
    return MOE_OK;
}
