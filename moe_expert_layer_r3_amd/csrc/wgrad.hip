// Weight-gradient grouped GEMM ("RL at 1T scale", section "FP8 Training":
// block-scaled FP8 trainer GEMMs; the backward re-quantises each operand along
// its contraction axis, here the token axis).
//
// For every local expert e and its padded row segment [offsets[e], offsets[e+1]):
//   dW[e][m, n] = sum over 128-row token blocks b of the segment of
//                 aT_s[m, b] * bT_s[n, b] * (aT[m, 128b:128b+128] . bT[n, 128b:128b+128])
// aT [M, row_cap] and bT [N, row_cap] are both K(=token)-contiguous, the layout
// the MFMA wants; scales are one per (row, token block) for both operands.
//
// Same machinery as the forward grouped GEMM (8 waves, 128 x 256 (or 128) tile,
// three-stage LDS DMA pipeline, conflict-free fragment layout); differences:
// the contraction runs over one expert's row segment (variable length, known
// only on the device), both operands carry per-row scales (the B scales of a
// stage are DMA'd next to the A scales), and the tile list is the dense
// (expert, m-tile, n-tile) grid, so experts without rows get dW = 0.
#include "mfma_common.hpp"

namespace moe {

constexpr int WBM = 128;
constexpr int WBK = 128;
constexpr int WTHREADS = 512;
constexpr int WWAVES = WTHREADS / 64;

struct WgradArgs {
    const uint8_t* aT;
    const float* aT_s;
    const uint8_t* bT;
    const float* bT_s;
    const int32_t* offsets;
    int L;
    int64_t row_cap;
    int M;
    int N;
    uint16_t* dW;
};

template <int BN>
struct WgradSmem {
    static constexpr int A_BYTES = WBM * WBK;
    static constexpr int B_BYTES = BN * WBK;
    static constexpr int SA_BYTES = WBM * 4;
    static constexpr int SB_BYTES = BN * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int TOTAL = 3 * STAGE;
};

template <int BN>
__global__ __launch_bounds__(WTHREADS, 1) void wgrad_fp8_kernel(WgradArgs g) {
    using SM = WgradSmem<BN>;
    constexpr int WN = BN / 4;
    constexpr int NI = WN / 16;
    constexpr int ASEG = WBM / 8 / WWAVES;  // 2
    constexpr int BSEG = BN / 8 / WWAVES;   // 4 (BN = 256) or 2
    constexpr int BROWS = BN / WWAVES;      // B rows (and B scales) loaded per wave
    constexpr int NLD = ASEG + BSEG + 2;    // + A scales + B scales

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t rcap = g.row_cap;
    const int MT = g.M / WBM, NT = g.N / BN;
    const int total = g.L * MT * NT;
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    const int l15 = lane & 15, l7 = lane & 7, c0 = lane >> 4;
    const uint32_t a_rd0 = (wm * 64 + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t a_rd1 = (wm * 64 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t b_rd0 = SM::A_BYTES + (wn * WN + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * WN + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t sa_rd = SM::A_BYTES + SM::B_BYTES + (wm * 64 + (lane >> 4) * 4) * 4;
    const uint32_t sb_rd = SM::A_BYTES + SM::B_BYTES + SM::SA_BYTES + (wn * WN + l15) * 4;

    for (int t = lb; t < total; t += G) {
        const int e = t / (MT * NT);
        const int rem = t - e * MT * NT;
        const int nt = rem / MT, mt = rem - nt * MT;  // m fastest: tiles in a row share bT
        int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
        if (lo > rcap) lo = rcap;
        if (hi > rcap) hi = rcap;
        const int nkb = __builtin_amdgcn_readfirstlane(hi > lo ? (int)((hi - lo) / WBK) : 0);
        const int64_t kb0 = lo / WBK;

        // DMA sources: rows of the transposed operands, K (= token) contiguous
        const int ra = wave * (ASEG * 8) + (lane >> 3);
        const uint8_t* a_src =
            g.aT + ((int64_t)mt * WBM + ra) * rcap + lo + (((lane & 7) ^ (ra & 7)) << 4);
        const int rb = wave * (BSEG * 8) + (lane >> 3);
        const uint8_t* b_src =
            g.bT + ((int64_t)nt * BN + rb) * rcap + lo + (((lane & 7) ^ (rb & 7)) << 4);
        // scales are token-block-major ([row_cap/128, M] and [row_cap/128, N]):
        // the rows of one token block are contiguous
        const float* sa_src = g.aT_s + kb0 * g.M + (int64_t)mt * WBM + wave * 16 + (lane & 15);
        const float* sb_src = g.bT_s + kb0 * g.N + (int64_t)nt * BN + wave * BROWS + (lane & (BROWS - 1));
        const int64_t R8 = 8 * rcap;

        auto issue = [&](int stage, int kb) {
            const uint32_t sA = sbase + (uint32_t)(stage * SM::STAGE);
            const uint32_t sB = sA + SM::A_BYTES;
            const uint32_t sSA = sB + SM::B_BYTES;
            const uint32_t sSB = sSA + SM::SA_BYTES;
            const int64_t kofs = (int64_t)kb * WBK;
#pragma unroll
            for (int i = 0; i < ASEG; ++i) dma16(a_src + i * R8 + kofs, sA + (wave * ASEG + i) * 1024);
#pragma unroll
            for (int i = 0; i < BSEG; ++i) dma16(b_src + i * R8 + kofs, sB + (wave * BSEG + i) * 1024);
            if (lane < 16) dma4(sa_src + (int64_t)kb * g.M, sSA + wave * 64);  // 16 A rows per wave
            if (lane < BROWS) dma4(sb_src + (int64_t)kb * g.N, sSB + wave * BROWS * 4);
        };

        v4f acc[4][NI];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

        __syncthreads();  // the previous tile's epilogue is done with smem
        if (nkb > 0) issue(0, 0);
        if (nkb > 1) issue(1, 1);
        for (int kb = 0; kb < nkb; ++kb) {
            if (kb + 1 < nkb) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            if (kb + 2 < nkb) issue((kb + 2) % 3, kb + 2);
            const uint32_t base = opaque(sbase + (uint32_t)((kb % 3) * SM::STAGE));

            u32x4 alo[4], ahi[4], sa4[4], blo[2], bhi[2];
            float sb[NI];
            blo[0] = lds16<0>(base + b_rd0);
            bhi[0] = lds16<0>(base + b_rd1);
            static_for<0, NI>([&](auto nc) {
                constexpr int ni = decltype(nc)::value;
                sb[ni] = __uint_as_float(*(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)(base + sb_rd + ni * 64));
            });
            static_for<0, 4>([&](auto ic) {
                constexpr int mi = decltype(ic)::value;
                alo[mi] = lds16<mi * 2048>(base + a_rd0);
                ahi[mi] = lds16<mi * 2048>(base + a_rd1);
                sa4[mi] = lds16<mi * 64>(base + sa_rd);
            });
            v8i af[4];
            v4f sa[4];
            v4f pt[2][4];
            const v8i bf0 = join8(blo[0], bhi[0]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                af[mi] = join8(alo[mi], ahi[mi]);
                sa[mi] = __builtin_bit_cast(v4f, sa4[mi]);
                pt[0][mi] = mfma16x16x128(af[mi], bf0);
            }
            static_for<0, NI + 1>([&](auto nc) {
                constexpr int ni = decltype(nc)::value;
                if constexpr (ni < NI) {
                    if constexpr (ni + 1 < NI) {
                        blo[(ni + 1) & 1] = lds16<(ni + 1) * 2048>(base + b_rd0);
                        bhi[(ni + 1) & 1] = lds16<(ni + 1) * 2048>(base + b_rd1);
                    }
                    if constexpr (ni > 0) {
                        const v8i bf = join8(blo[ni & 1], bhi[ni & 1]);
#pragma unroll
                        for (int mi = 0; mi < 4; ++mi) pt[ni & 1][mi] = mfma16x16x128(af[mi], bf);
                    }
                }
                if constexpr (ni > 0) {
                    constexpr int pn = ni - 1;
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) acc[mi][pn] += pt[pn & 1][mi] * (sa[mi] * sb[pn]);
                }
            });
        }
        __syncthreads();

        // bf16 store through an LDS staging tile
        constexpr int LDR = BN * 2 + 16;
        static_assert(WBM * LDR <= SM::TOTAL, "staging fits");
        const int rbase = wm * 64 + (lane >> 4) * 4;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rbase + mi * 16 + i;
                    const int c = wn * WN + ni * 16 + l15;
                    *reinterpret_cast<uint16_t*>(smem + r * LDR + c * 2) = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                }
        __syncthreads();
        uint16_t* out = g.dW + (int64_t)e * g.M * g.N + (int64_t)mt * WBM * g.N + (int64_t)nt * BN;
        constexpr int CPR = BN / 8;
        for (int idx = tid; idx < WBM * CPR; idx += WTHREADS) {
            const int r = idx / CPR, ch = idx - r * CPR;
            const uint4 v = *reinterpret_cast<const uint4*>(smem + r * LDR + ch * 16);
            *reinterpret_cast<uint4*>(out + (int64_t)r * g.N + ch * 8) = v;
        }
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_gemm_fp8_wgrad(const uint8_t* aT, const float* aT_s, const uint8_t* bT,
                                          const float* bT_s, const int32_t* offsets, int32_t L, int64_t row_cap,
                                          int32_t M, int32_t N, uint16_t* dW, hipStream_t stream) {
    MOE_REQUIRE(L >= 1 && L <= 1024, MOE_ERR_SHAPE, "grouped_gemm_wgrad: L=%d outside [1, 1024]", L);
    MOE_REQUIRE(row_cap >= 0 && row_cap % WBK == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(M > 0 && M % WBM == 0 && N > 0 && N % 128 == 0, MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: M=%d and N=%d must be multiples of 128", M, N);
    MOE_REQUIRE((int64_t)L * (M / WBM) * (N / 128) < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: too many tiles");
    MOE_REQUIRE(aT && aT_s && bT && bT_s && offsets && dW, MOE_ERR_NULL, "grouped_gemm_wgrad: NULL argument");
    WgradArgs a{aT, aT_s, bT, bT_s, offsets, L, row_cap, M, N, dW};
    const int grid = (num_cus() + 7) / 8 * 8;  // persistent, one block per CU
    if (N % 256 == 0)
        wgrad_fp8_kernel<256><<<dim3(grid), dim3(WTHREADS), 0, stream>>>(a);
    else
        wgrad_fp8_kernel<128><<<dim3(grid), dim3(WTHREADS), 0, stream>>>(a);
    MOE_LAUNCH_CHECK("wgrad_fp8_kernel");
    return MOE_OK;
}
