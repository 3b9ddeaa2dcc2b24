// Weight-gradient grouped GEMM ("RL at 1T scale", section "FP8 Training":
// block-scaled FP8 trainer GEMMs; the backward re-quantises each operand along
// its contraction axis, here the token axis).
//
// For every local expert e and its padded row segment [offsets[e], offsets[e+1]):
//   dW[e][m, n] = sum over 128-row token blocks b of the segment of
//                 aT_s[b, m] * bT_s[b, n] * (aT[m, 128b:128b+128] . bT[n, 128b:128b+128])
// aT [M, row_cap] and bT [N, row_cap] are both K(=token)-contiguous, the layout
// the MFMA wants; scales are one per (row, token block) for both operands and
// stored token-block-major, so one block's scales of a tile are contiguous.
//
// Same machinery as the forward grouped GEMM (8 waves in two ping-pong groups,
// 128 x 128 tile, three-stage LDS DMA ring, conflict-free fragment
// layout, weights-first MFMA operand order, register-direct epilogue with the
// next tile's first stages already in flight); differences: the contraction
// runs over one expert's row segment (variable length, known only on the
// device, possibly empty), both operands carry per-row scales (the factor of
// a partial is sA[row] * sB[column], formed as the partial is added), and the
// tile list is the dense (expert, m-tile, n-tile) grid, so experts without
// rows get dW = 0.
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
    constexpr int WN = BN / 4;              // wave tile columns
    constexpr int NI = WN / 16;             // n-subtiles per wave
    constexpr int ASEG = WBM / 8 / WWAVES;  // 1 KB A segments per wave (2)
    constexpr int BSEG = BN / 8 / WWAVES;   // 1 KB B segments per wave (4 or 2)
    constexpr int BROWS = BN / WWAVES;      // B rows (and B scales) loaded per wave
    constexpr int NLD = ASEG + BSEG + 2;    // DMA instructions per wave per stage (+ A and B scales)

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t rcap = g.row_cap;
    const int M = g.M, N = g.N;
    const int MT = M / WBM, NT = N / BN;
    const int total = g.L * MT * NT;
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // fragment read offsets (lane l: row l & 15 of a fragment, K chunks g and
    // g + 4 of the 128-byte block, g = l >> 4; swizzled chunk c ^ (row & 7))
    const int l15 = lane & 15, l7 = lane & 7, c0 = lane >> 4, lg = lane >> 4;
    const uint32_t a_rd0 = (wm * 64 + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t a_rd1 = (wm * 64 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t b_rd0 = SM::A_BYTES + (wn * WN + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * WN + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    // A scales: the 16 bytes at slot wm*64 + 4*l15 hold rows wm*64 + mi*16 + l15
    // (mi = 0..3); B scales: natural order, 4 consecutive columns per read
    const uint32_t sa_rd = SM::A_BYTES + SM::B_BYTES + (wm * 64 + l15 * 4) * 4;
    const uint32_t sb_rd = SM::A_BYTES + SM::B_BYTES + SM::SA_BYTES + (wn * WN + 4 * lg) * 4;
    uint32_t rA0[3], rA1[3], rB0[3], rB1[3], rSA[3], rSB[3];
#pragma unroll
    for (int st = 0; st < 3; ++st) {
        const uint32_t b = sbase + (uint32_t)(st * SM::STAGE);
        rA0[st] = b + a_rd0;
        rA1[st] = b + a_rd1;
        rB0[st] = b + b_rd0;
        rB1[st] = b + b_rd1;
        rSA[st] = b + sa_rd;
        rSB[st] = b + sb_rd;
    }

    struct Tile {
        int e, mt, nt, nkb;
        const uint8_t* a_base;   // this wave's first A row at the segment start
        const uint8_t* b_base;
        const float* sa_base;    // the tile's A scales, first token block of the segment
        const float* sb_base;    // this wave's B scales, first token block
    };
    auto tile_at = [&](int t) {
        Tile ti;
        ti.e = t / (MT * NT);
        const int rem = t - ti.e * MT * NT;
        ti.nt = rem / MT;  // m fastest: consecutive tiles share the B operand
        ti.mt = rem - ti.nt * MT;
        int64_t lo = g.offsets[ti.e], hi = g.offsets[ti.e + 1];
        if (lo > rcap) lo = rcap;
        if (hi > rcap) hi = rcap;
        ti.nkb = __builtin_amdgcn_readfirstlane(hi > lo ? (int)((hi - lo) / WBK) : 0);
        const int64_t kb0 = lo / WBK;
        ti.a_base = g.aT + ((int64_t)ti.mt * WBM + wave * ASEG * 8) * rcap + lo;
        ti.b_base = g.bT + ((int64_t)ti.nt * BN + wave * BSEG * 8) * rcap + lo;
        ti.sa_base = g.aT_s + kb0 * M + (int64_t)ti.mt * WBM;
        ti.sb_base = g.bT_s + kb0 * N + (int64_t)ti.nt * BN + wave * BROWS;
        return ti;
    };

    // DMA lane offsets (swizzled chunk of row 8q + l/8 of each 1 KB segment)
    const int lr = lane >> 3;
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ lr) << 4);
    uint32_t a_off[ASEG], b_off[BSEG];
#pragma unroll
    for (int i = 0; i < ASEG; ++i) a_off[i] = (uint32_t)((8 * i + lr) * rcap) + chunk;
#pragma unroll
    for (int i = 0; i < BSEG; ++i) b_off[i] = (uint32_t)((8 * i + lr) * rcap) + chunk;
    // lane l < 16 of wave w fills A scale slot w*16 + l: row (w/4)*64 + (l%4)*16
    // + (w%4)*4 + l/4 (the slot layout above)
    const uint32_t sa_off = (uint32_t)(((wave >> 2) * 64 + (lane & 3) * 16 + (wave & 3) * 4 + ((lane & 15) >> 2)) * 4);
    const uint32_t sb_off = (uint32_t)((lane & (BROWS - 1)) * 4);

    auto issue = [&](auto stage_c, int kb, const Tile& ti) {
        constexpr int stage = decltype(stage_c)::value;
        const uint32_t sA = sbase + (uint32_t)(stage * SM::STAGE);
        const uint32_t sB = sA + SM::A_BYTES;
        const uint32_t sSA = sB + SM::B_BYTES;
        const uint32_t sSB = sSA + SM::SA_BYTES;
        const int64_t kofs = (int64_t)kb * WBK;
#pragma unroll
        for (int i = 0; i < ASEG; ++i) dma16s(ti.a_base + kofs, a_off[i], sA + (wave * ASEG + i) * 1024);
#pragma unroll
        for (int i = 0; i < BSEG; ++i) dma16s(ti.b_base + kofs, b_off[i], sB + (wave * BSEG + i) * 1024);
        if (lane < 16) dma4s(ti.sa_base + (int64_t)kb * M, sa_off, sSA + wave * 64);
        if (lane < BROWS) dma4s(ti.sb_base + (int64_t)kb * N, sb_off, sSB + wave * BROWS * 4);
    };
    auto lds_barrier = [&]() {
        wait_lgkm0();
        phase_barrier();
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    int t = lb;
    Tile cur;
    if (t < total) {
        cur = tile_at(t);
        if (cur.nkb > 0) issue(S0{}, 0, cur);
        if (cur.nkb > 1) issue(S1{}, 1, cur);
    }
    for (; t < total; t += G) {
        const int nkb = cur.nkb;
        v4f acc[4][NI];
        v8i af[4], bfr[NI];
        float sa[4];          // A scales of the loaded block (rows of this lane)
        v4f sb[NI];           // B scales of the loaded block (4 columns per n-subtile)
        v4f ring[4];          // raw partials awaiting their rescale
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;
            ring[mi] = zero4;
            sa[mi] = 0.f;
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) sb[ni] = zero4;

        auto flush = [&]() {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][NI - 1] += ring[mi] * (sa[mi] * sb[NI - 1]);
        };
        auto load = [&](auto stage_c) {
            constexpr int st = decltype(stage_c)::value;
            const uint32_t pa0 = opaque(rA0[st]), pa1 = opaque(rA1[st]);
            const uint32_t pb0 = opaque(rB0[st]), pb1 = opaque(rB1[st]);
            const uint32_t psa = opaque(rSA[st]), psb = opaque(rSB[st]);
            const u32x4 sa4 = lds16<0>(psa);
            u32x4 sbn[NI];
            static_for<0, NI>([&](auto nc) {
                constexpr int ni = decltype(nc)::value;
                sbn[ni] = lds16<ni * 64>(psb);
            });
            static_for<0, 4>([&](auto ic) {
                constexpr int mi = decltype(ic)::value;
                af[mi] = join8(lds16<mi * 2048>(pa0), lds16<mi * 2048>(pa1));
            });
            static_for<0, NI>([&](auto nc) {
                constexpr int ni = decltype(nc)::value;
                bfr[ni] = join8(lds16<ni * 2048>(pb0), lds16<ni * 2048>(pb1));
            });
            flush();  // with the previous block's scales
            const uint32_t sav[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) sa[mi] = __uint_as_float(sav[mi]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) sb[ni] = __builtin_bit_cast(v4f, sbn[ni]);
            wait_lgkm0();
        };
        auto compute = [&]() {
            static_for<0, 4 * NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int ni = j / 4, mi = j % 4;
                if constexpr (j >= 4) acc[mi][ni - 1] += ring[mi] * (sa[mi] * sb[ni - 1]);
                ring[mi] = mfma16x16x128(bfr[ni], af[mi]);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto step0 = [&](auto st_c, int kb) {
            constexpr int st = decltype(st_c)::value;
            if (kb + 1 < nkb) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
            phase_barrier();
            if (kb + 2 < nkb) issue(std::integral_constant<int, (st + 2) % 3>{}, kb + 2, cur);
            load(st_c);
            phase_barrier();
            compute();
        };
        auto step1 = [&](auto st_c, int kb) {
            constexpr int st = decltype(st_c)::value;
            if (kb + 1 < nkb) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
            phase_barrier();
            if (kb + 2 < nkb) issue(std::integral_constant<int, (st + 2) % 3>{}, kb + 2, cur);
            compute();
            phase_barrier();
            load(st_c);
        };
        if (nkb > 0) {
            if (wave < 4) {
                for (int kb = 0; kb < nkb; kb += 3) {
                    step0(S0{}, kb);
                    if (kb + 1 < nkb) step0(S1{}, kb + 1);
                    if (kb + 2 < nkb) step0(S2{}, kb + 2);
                }
            } else {
                if (nkb > 1) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
                phase_barrier();
                if (nkb > 2) issue(S2{}, 2, cur);
                phase_barrier();
                load(S0{});
                for (int kb = 1; kb < nkb; kb += 3) {
                    step1(S1{}, kb);
                    if (kb + 1 < nkb) step1(S2{}, kb + 1);
                    if (kb + 2 < nkb) step1(S0{}, kb + 2);
                }
                compute();
            }
            flush();
        }
        // stages free: the next tile's first two stages go out before this
        // tile's epilogue
        lds_barrier();
        const Tile ep = cur;
        if (t + G < total) {
            cur = tile_at(t + G);
            if (cur.nkb > 0) issue(S0{}, 0, cur);
            if (cur.nkb > 1) issue(S1{}, 1, cur);
        }
        // bf16 store straight from registers: row wm*64 + mi*16 + l15, columns
        // wn*WN + ni*16 + 4*lg + v of the tile
        uint16_t* out = g.dW + (int64_t)ep.e * M * N + (int64_t)ep.mt * WBM * N + (int64_t)ep.nt * BN;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int64_t r = wm * 64 + mi * 16 + l15;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const v4f a = acc[mi][ni];
                *reinterpret_cast<v2u*>(out + r * N + wn * WN + ni * 16 + 4 * lg) =
                    v2u{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w)};
            }
        }
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_gemm_fp8_wgrad(const uint8_t* aT, const float* aT_s, const uint8_t* bT,
                                          const float* bT_s, const int32_t* offsets, int32_t L, int64_t row_cap,
                                          int32_t M, int32_t N, uint16_t* dW, hipStream_t stream) {
    MOE_REQUIRE(L >= 1 && L <= 1024, MOE_ERR_SHAPE, "grouped_gemm_wgrad: L=%d outside [1, 1024]", L);
    // lane offsets into the operand rows are 32-bit: 16 rows of row_cap bytes must fit
    MOE_REQUIRE(row_cap >= 0 && row_cap % WBK == 0 && row_cap < ((int64_t)1 << 28), MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: row_cap=%lld must be a multiple of 128 below 2^28", (long long)row_cap);
    MOE_REQUIRE(M > 0 && M % WBM == 0 && N > 0 && N % 128 == 0, MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: M=%d and N=%d must be multiples of 128", M, N);
    MOE_REQUIRE((int64_t)L * (M / WBM) * (N / 128) < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: too many tiles");
    MOE_REQUIRE(aT && aT_s && bT && bT_s && offsets && dW, MOE_ERR_NULL, "grouped_gemm_wgrad: NULL argument");
    WgradArgs a{aT, aT_s, bT, bT_s, offsets, L, row_cap, M, N, dW};
    const int grid = (num_cus() + 7) / 8 * 8;  // persistent, one block per CU
    // 128 x 128 tiles only: with both operands scaled per row, a 128 x 256
    // tile needs more than 256 VGPRs and spills inside the K loop, which costs
    // more than the extra A traffic of the narrower tile (measured 1.75x slower)
    wgrad_fp8_kernel<128><<<dim3(grid), dim3(WTHREADS), 0, stream>>>(a);
    MOE_LAUNCH_CHECK("wgrad_fp8_kernel");
    return MOE_OK;
}
