// MXFP4 quantisation of expert weights (OCP Microscaling v1.0 FP4: E2M1
// elements, one E8M0 power-of-two scale per 32 consecutive values along K).
// The pages name 4-bit training and inference as future work ("RL at 1T
// scale", section on future work); MXFP4 is the 4-bit block format that
// gfx950's block-scaled matrix instruction applies natively.
//
// Per block of 32 values V:  E = floor(log2(max|V|)) - 2, clamped to
// [-127, 127] (-127 for an all-zero block; 2 is the exponent of E2M1's largest
// normal 6 = 1.5 * 2^2), scale code E + 127, and each value's code is the
// nearest E2M1 magnitude of |V_i| * 2^-E (ties to the even code, above 6
// clamped to 6) with the sign bit of V_i.
#include "common.hpp"

namespace moe {

// Eight already-scaled values (v * 2^-E, exact) to eight E2M1 codes, value i
// in bits 4i .. 4i+3.  gfx950's v_cvt_scalef32_pk_fp4_f32 rounds x / s to the
// nearest E2M1 value with ties to the even code, saturates at 6 and keeps the
// sign (measured against that definition on a dense sweep of [-10, 10],
// signed zeros included); with s = 1 it does only the rounding, so blocks
// whose scale 2^-127 is not a normal float need no special case.  The first
// operand of a pair goes to the low nibble; the last argument picks the byte.
__device__ __forceinline__ uint32_t e2m1_pack8(const float x[8]) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[0], x[1], 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[2], x[3], 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[4], x[5], 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[6], x[7], 1.0f, 3);
    return r;
}

// One thread per 8 values (one 16-byte load); the 4 threads of a 32-block
// agree on its maximum through two xor shuffles.  Every value is exact in
// fp32 (bf16 source), the maximum's exponent field gives floor(log2), and
// v * 2^-E is exact, so the codes match the definition bit for bit.
// Codes and scales are stored K-block-major per group, [groups, cols/128,
// rows, 64] and [groups, cols/128, rows, 4]: a GEMM K step reads 64 code bytes
// and 4 scale bytes of each of a tile's rows, and this way a K step of
// consecutive rows is contiguous.  Row-major layouts cost one cache-line
// request per row and K step for half a line of codes and 4 scale bytes.
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                           int64_t nrows, int64_t cols, int64_t ld,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int64_t per_row = cols >> 3;
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= nrows * per_row) return;  // whole 4-thread groups leave together (per_row % 4 == 0)
    const int64_t r = item / per_row, c8 = (item - r * per_row) * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(src + r * ld + c8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = group_max<4>(am);
    const int ef = (int)((__float_as_uint(am) >> 23) & 0xFFu);  // 0 for zero and subnormal maxima
    const int code = ef == 0 ? 0 : max(ef - 2, 0);                  // E + 127 with E = ef - 129 >= -127
    const float inv = __uint_as_float((uint32_t)(254 - code) << 23); // 2^-E
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = v[i] * inv;
    const uint32_t packed = e2m1_pack8(x);
    const int64_t g = r / rows, rr = r - g * rows;
    const int64_t blk = (g * (cols >> 7) + (c8 >> 7)) * rows + rr;  // (group, K block, row)
    *reinterpret_cast<uint32_t*>(q + blk * 64 + ((c8 & 127) >> 1)) = packed;
    if ((c8 & 31) == 0) s[blk * 4 + ((c8 >> 5) & 3)] = (uint8_t)code;
}

// Both quantisations of a weight matrix in one pass, for training: blocks along
// columns (the forward product's K) and blocks along rows (the dgrad product,
// which reads the transpose).  One block of 256 threads per 128 x 128 tile;
// thread (wave w, lane l) holds rows 8*rq .. 8*rq + 7, rq = 4w + l/16, and
// columns 8*cg .. 8*cg + 7, cg = l % 16:
//   * a row's 32-column block is 4 neighbouring lanes (cg ^ 1, ^ 2);
//   * a column's 32-row block is wave w's four row octets (lanes 16 apart).
// Codes of both layouts are assembled in LDS and leave as whole 64-byte
// records (a record = one row's, resp. one column's, 128 codes of the tile).
__global__ __launch_bounds__(256) void quant_mxfp4_both_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                                int64_t cols, int64_t ld, uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s, uint8_t* __restrict__ qT,
                                                                uint8_t* __restrict__ sT) {
    __shared__ __attribute__((aligned(16))) uint8_t rec[2][128][64 + 16];
    __shared__ __attribute__((aligned(16))) uint8_t srec[2][128][4];
    const int64_t g = blockIdx.z, rb = blockIdx.y, cb = blockIdx.x;
    const int64_t rbn = rows >> 7, cbn = cols >> 7;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = wave * 4 + (lane >> 4);
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint4 raw =
            *reinterpret_cast<const uint4*>(src + (g * rows + rb * 128 + rq * 8 + j) * ld + cb * 128 + cg * 8);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[j][2 * i] = bf16_lo(w4[i]);
            v[j][2 * i + 1] = bf16_hi(w4[i]);
        }
    }
    // blocks along columns: row 8rq + j, columns 32*(cg/4) .. +31
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[j][i]));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        const int ef = (int)((__float_as_uint(am) >> 23) & 0xFFu);
        const int code = ef == 0 ? 0 : max(ef - 2, 0);
        const float inv = __uint_as_float((uint32_t)(254 - code) << 23);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = v[j][i] * inv;
        *reinterpret_cast<uint32_t*>(&rec[0][rq * 8 + j][cg * 4]) = e2m1_pack8(x);
        if ((cg & 3) == 0) srec[0][rq * 8 + j][cg >> 2] = (uint8_t)code;
    }
    // blocks along rows: column 8cg + i, rows 32*w .. +31
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(v[j][i]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        const int ef = (int)((__float_as_uint(am) >> 23) & 0xFFu);
        const int code = ef == 0 ? 0 : max(ef - 2, 0);
        const float inv = __uint_as_float((uint32_t)(254 - code) << 23);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = v[j][i] * inv;
        *reinterpret_cast<uint32_t*>(&rec[1][cg * 8 + i][rq * 4]) = e2m1_pack8(x);
        if ((lane >> 4) == 0) srec[1][cg * 8 + i][wave] = (uint8_t)code;
    }
    __syncthreads();
    // 128 records of 64 bytes per layout: 512 16-byte pieces, 2 per thread
    uint8_t* const qo = q + ((g * cbn + cb) * rows + rb * 128) * 64;    // records: rows of this tile, K block cb
    uint8_t* const to = qT + ((g * rbn + rb) * cols + cb * 128) * 64;   // records: columns of this tile, K block rb
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int k = tid + 256 * m, r = k >> 2, part = (k & 3) * 16;
        *reinterpret_cast<uint4*>(qo + r * 64 + part) = *reinterpret_cast<const uint4*>(&rec[0][r][part]);
        *reinterpret_cast<uint4*>(to + r * 64 + part) = *reinterpret_cast<const uint4*>(&rec[1][r][part]);
    }
    if (tid < 128) {
        *reinterpret_cast<uint32_t*>(s + ((g * cbn + cb) * rows + rb * 128 + tid) * 4) =
            *reinterpret_cast<const uint32_t*>(&srec[0][tid][0]);
    } else {
        const int c = tid - 128;
        *reinterpret_cast<uint32_t*>(sT + ((g * rbn + rb) * cols + cb * 128 + c) * 4) =
            *reinterpret_cast<const uint32_t*>(&srec[1][c][0]);
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_quant_mxfp4(const uint16_t* src, int64_t groups, int64_t rows, int64_t cols, int64_t ld,
                               uint8_t* q, uint8_t* scales, uint8_t* qT, uint8_t* scalesT, hipStream_t stream) {
    MOE_REQUIRE(groups >= 0 && rows >= 0 && cols >= 0 && cols % 128 == 0, MOE_ERR_SHAPE,
                "quant_mxfp4: cols=%lld must be a multiple of 128", (long long)cols);
    MOE_REQUIRE(ld >= cols && ld % 8 == 0, MOE_ERR_SHAPE, "quant_mxfp4: ld=%lld must be >= cols and a multiple of 8",
                (long long)ld);
    MOE_REQUIRE(!qT == !scalesT, MOE_ERR_NULL, "quant_mxfp4: qT and scalesT go together");
    MOE_REQUIRE(!qT || rows % 128 == 0, MOE_ERR_SHAPE, "quant_mxfp4: the transposed copy needs rows %% 128 == 0");
    if (groups == 0 || rows == 0 || cols == 0) return MOE_OK;
    MOE_REQUIRE(src && q && scales, MOE_ERR_NULL, "quant_mxfp4: NULL src/q/scales");
    if (qT) {
        MOE_REQUIRE(rows / 128 <= 65535 && groups <= 65535, MOE_ERR_SHAPE, "quant_mxfp4: too many tiles");
        dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128), (unsigned)groups);
        quant_mxfp4_both_kernel<<<grid, dim3(256), 0, stream>>>(src, rows, cols, ld, q, scales, qT, scalesT);
        MOE_LAUNCH_CHECK("quant_mxfp4_both_kernel");
        return MOE_OK;
    }
    const int64_t nrows = groups * rows;
    const int64_t threads = nrows * (cols / 8);
    MOE_REQUIRE((threads + 255) / 256 <= 0x7FFFFFFF, MOE_ERR_SHAPE, "quant_mxfp4: too large");
    quant_mxfp4_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(src, rows, nrows, cols,
                                                                                       ld, q, scales);
    MOE_LAUNCH_CHECK("quant_mxfp4_kernel");
    return MOE_OK;
}
