// Backward through the SwiGLU expert activation, with the FP8 re-quantisation
// of its results for the next GEMMs ("RL at 1T scale", section "FP8 Training":
// every backward GEMM operand is block-quantised along that GEMM's contraction
// axis).
//
// For a row r of the expert-grouped layout and a column c < f, from the GEMM
// result dH (fp32) and the saved bf16 pre-activations G = GU[:, :f], U = GU[:, f:]:
//     s  = 1 / (1 + exp(-G))      (hardware exp2 and reciprocal, about 1 ulp)
//     dG = dH * U * s * (1 + G * (1 - s))      (derivative of silu(G) * U in G)
//     dU = dH * G * s                          (silu(G) = G * s)
//     H  = G * s * U                           (the activation, recomputed)
// all in fp32.  Outputs: [dG, dU] quantised 1x128 along features (operand of the
// dgrad GEMM through W13) and 128x1 along rows, transposed (operand of the W13
// weight gradient); H quantised 128x1 transposed (operand of the W2 weight
// gradient).  Padding rows (row_pair < 0) count as zero in the 128x1 tiles and
// are not written in the row-major outputs.
#include "common.hpp"

namespace moe {

struct SwigluBwdArgs {
    const float* dH;
    const uint16_t* gu;
    const int32_t* row_pair;
    const int32_t* offsets;
    int L;
    int64_t row_cap;
    int f;
    uint8_t* dgu_q;
    float* dgu_s;
    uint8_t* dgu_qT;
    float* dgu_sT;
    uint8_t* h_qT;
    float* h_sT;
    float* dgu_f32;
    float* h_f32;
};

// One block per (128-row block, 128-column block of f), the column block the
// grid's fast index; 256 threads.  Thread
// (wave w, lane l) covers rows 8*rq .. 8*rq + 7 of the block, rq = 4w + l/16,
// and columns 8*cg .. +7 of the f-block, cg = l % 16, for all three results:
//   * the 16 lanes of a row share its 1x128 tiles (a 16-lane max);
//   * a column's maximum over the block's 128 rows is the thread's 8 rows, the
//     wave's 4 row octets (lanes 16 apart), then the 4 waves through a small
//     LDS array;
//   * a column's codes for the thread's 8 consecutive rows are one 8-byte word
//     of the transposed LDS tile, which leaves as 16-byte stores of full
//     128-byte columns.
template <bool P2>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(SwigluBwdArgs a) {
    __shared__ __attribute__((aligned(16))) float cmax[3][4][128];
    __shared__ __attribute__((aligned(16))) uint8_t tile_t[3][128][128 + 8];
    // column blocks fastest: workgroups launched together take neighbouring
    // column blocks of the same rows
    const int64_t b = blockIdx.y, cb = blockIdx.x;
    int64_t total = a.offsets[a.L];
    if (total > a.row_cap) total = a.row_cap;
    if (b * 128 >= total) return;  // whole block leaves together
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = lane & 15, rq = wave * 4 + (lane >> 4);
    const int c8 = cg * 8;
    const int f = a.f;
    const int64_t F2 = 2 * (int64_t)f;
    const int64_t col = cb * 128 + c8;  // column of f
    const int64_t r0 = b * 128 + rq * 8;
    const int4* rp = reinterpret_cast<const int4*>(a.row_pair + r0);
    const int4 pa = rp[0], pb = rp[1];
    const bool real[8] = {pa.x >= 0, pa.y >= 0, pa.z >= 0, pa.w >= 0, pb.x >= 0, pb.y >= 0, pb.z >= 0, pb.w >= 0};

    float dg[8][8], du[8][8], hh[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = r0 + j;
        if (real[j]) {
            const float4* hp = reinterpret_cast<const float4*>(a.dH + r * f + col);
            const float4 h0 = hp[0], h1 = hp[1];
            const float dh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            const uint4 gr = *reinterpret_cast<const uint4*>(a.gu + r * F2 + col);
            const uint4 ur = *reinterpret_cast<const uint4*>(a.gu + r * F2 + f + col);
            const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
            const uint32_t uw[4] = {ur.x, ur.y, ur.z, ur.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float g = (i & 1) ? bf16_hi(gw[i >> 1]) : bf16_lo(gw[i >> 1]);
                const float u = (i & 1) ? bf16_hi(uw[i >> 1]) : bf16_lo(uw[i >> 1]);
                const float s = sigmoid_fast(g);
                const float gs = g * s;
                dg[j][i] = dh[i] * u * s * (1.0f + g * (1.0f - s));
                du[j][i] = dh[i] * gs;
                hh[j][i] = gs * u;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) dg[j][i] = du[j][i] = hh[j][i] = 0.f;
        }
    }

    // row-major outputs: 1x128 [dG, dU] (the 16 lanes of a row share the tile)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = r0 + j;
        float mg = 0.f, mu = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mg = fmaxf(mg, fabsf(dg[j][i]));
            mu = fmaxf(mu, fabsf(du[j][i]));
        }
        mg = group_max<16>(mg);
        mu = group_max<16>(mu);
        if (!real[j]) continue;
        const TileScale tg = tile_scale_t<P2>(mg), tu = tile_scale_t<P2>(mu);
        uint2 qg, qu;
        qg.x = cvt_e4m3x4(dg[j][0] * tg.inv, dg[j][1] * tg.inv, dg[j][2] * tg.inv, dg[j][3] * tg.inv);
        qg.y = cvt_e4m3x4(dg[j][4] * tg.inv, dg[j][5] * tg.inv, dg[j][6] * tg.inv, dg[j][7] * tg.inv);
        qu.x = cvt_e4m3x4(du[j][0] * tu.inv, du[j][1] * tu.inv, du[j][2] * tu.inv, du[j][3] * tu.inv);
        qu.y = cvt_e4m3x4(du[j][4] * tu.inv, du[j][5] * tu.inv, du[j][6] * tu.inv, du[j][7] * tu.inv);
        *reinterpret_cast<uint2*>(a.dgu_q + r * F2 + col) = qg;
        *reinterpret_cast<uint2*>(a.dgu_q + r * F2 + f + col) = qu;
        if (cg == 0) {
            a.dgu_s[cb * a.row_cap + r] = tg.s;  // K-block-major scales
            a.dgu_s[((f >> 7) + cb) * a.row_cap + r] = tu.s;
        }
        if (a.dgu_f32) {
            float4* pg = reinterpret_cast<float4*>(a.dgu_f32 + r * F2 + col);
            float4* pu = reinterpret_cast<float4*>(a.dgu_f32 + r * F2 + f + col);
            pg[0] = make_float4(dg[j][0], dg[j][1], dg[j][2], dg[j][3]);
            pg[1] = make_float4(dg[j][4], dg[j][5], dg[j][6], dg[j][7]);
            pu[0] = make_float4(du[j][0], du[j][1], du[j][2], du[j][3]);
            pu[1] = make_float4(du[j][4], du[j][5], du[j][6], du[j][7]);
        }
        if (a.h_f32) {
            float4* ph = reinterpret_cast<float4*>(a.h_f32 + r * f + col);
            ph[0] = make_float4(hh[j][0], hh[j][1], hh[j][2], hh[j][3]);
            ph[1] = make_float4(hh[j][4], hh[j][5], hh[j][6], hh[j][7]);
        }
    }

    // 128x1 tiles: column maxima over the block's 128 rows
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        float am[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(q == 0 ? dg[j][i] : q == 1 ? du[j][i] : hh[j][i]));
            m = fmaxf(m, __shfl_xor(m, 16));
            am[i] = fmaxf(m, __shfl_xor(m, 32));
        }
        if (lane < 16) {
            *reinterpret_cast<float4*>(&cmax[q][wave][c8]) = make_float4(am[0], am[1], am[2], am[3]);
            *reinterpret_cast<float4*>(&cmax[q][wave][c8 + 4]) = make_float4(am[4], am[5], am[6], am[7]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float m = fmaxf(fmaxf(cmax[q][0][c8 + i], cmax[q][1][c8 + i]),
                                  fmaxf(cmax[q][2][c8 + i], cmax[q][3][c8 + i]));
            const TileScale ts = tile_scale_t<P2>(m);
            if (wave == 0 && lane < 16) {
                // scales of the transposed tiles, token-block-major: dG at
                // column c, dU at f + c (of 2f), H at c (of f)
                float* sT = q == 2 ? a.h_sT : a.dgu_sT;
                const int64_t c = (q == 1 ? f : 0) + col + i;
                sT[b * (q == 2 ? (int64_t)f : F2) + c] = ts.s;
            }
            // column c8 + i, rows 8rq .. 8rq + 7: bytes 0..7 of one word
            const float x = ts.inv;
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = (q == 0 ? dg[j][i] : q == 1 ? du[j][i] : hh[j][i]) * x;
            const uint32_t lo = cvt_e4m3x4(y[0], y[1], y[2], y[3]);
            const uint32_t hi = cvt_e4m3x4(y[4], y[5], y[6], y[7]);
            *reinterpret_cast<uint2*>(&tile_t[q][c8 + i][rq * 8]) = make_uint2(lo, hi);
        }
    __syncthreads();
    for (int idx = tid; idx < 3 * 128 * 8; idx += 256) {
        const int q = idx >> 10, c = (idx >> 3) & 127, part = (idx & 7) * 16;
        const uint4 val = *reinterpret_cast<const uint4*>(&tile_t[q][c][part]);
        uint8_t* dst = q == 2 ? a.h_qT : a.dgu_qT;
        const int64_t crow = (q == 1 ? f : 0) + cb * 128 + c, C = q == 2 ? (int64_t)f : F2;
        *reinterpret_cast<uint4*>(dst + ((b * C + crow) << 7) + part) = val;
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_swiglu_backward(const float* dH, const uint16_t* gu, const int32_t* row_pair,
                                   const int32_t* offsets, int32_t L, int64_t row_cap, int32_t f,
                                   uint8_t* dgu_q, float* dgu_s, uint8_t* dgu_qT, float* dgu_sT, uint8_t* h_qT,
                                   float* h_sT, float* dgu_f32, float* h_f32, int32_t flags, hipStream_t stream) {
    MOE_REQUIRE(flags == 0 || flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED, "swiglu_backward: unknown flags 0x%x", flags);
    MOE_REQUIRE(L >= 1 && L <= 1024, MOE_ERR_SHAPE, "swiglu_backward: L=%d outside [1, 1024]", L);
    MOE_REQUIRE(row_cap >= 0 && row_cap % 128 == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "swiglu_backward: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(f > 0 && f % 128 == 0 && f / 128 <= 65535, MOE_ERR_SHAPE,
                "swiglu_backward: f=%d must be a positive multiple of 128", f);
    MOE_REQUIRE(dH && gu && row_pair && offsets && dgu_q && dgu_s && dgu_qT && dgu_sT && h_qT && h_sT,
                MOE_ERR_NULL, "swiglu_backward: NULL argument");
    if (row_cap == 0) return MOE_OK;
    SwigluBwdArgs args{dH, gu, row_pair, offsets, L, row_cap, f, dgu_q, dgu_s, dgu_qT, dgu_sT,
                       h_qT, h_sT, dgu_f32, h_f32};
    MOE_REQUIRE(row_cap / 128 <= 65535, MOE_ERR_SHAPE, "swiglu_backward: row_cap too large");
    const dim3 grid((unsigned)(f / 128), (unsigned)(row_cap / 128));
    if (flags)
        swiglu_bwd_kernel<true><<<grid, 256, 0, stream>>>(args);
    else
        swiglu_bwd_kernel<false><<<grid, 256, 0, stream>>>(args);
    MOE_LAUNCH_CHECK("swiglu_bwd_kernel");
    return MOE_OK;
}
