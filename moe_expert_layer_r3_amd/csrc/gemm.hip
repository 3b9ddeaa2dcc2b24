// Block-scaled FP8 grouped GEMM on gfx950 MFMA ("RL at 1T scale", section "FP8
// Training": block-scaled FP8 trainer GEMMs in the DeepSeek-V3 style).
//
// C[r, n] = sum_c sA[r, c] * sB[n/128, c] * (A[r, 128c:128c+128] . B[n, 128c:128c+128])
// for the real rows r of each expert's 128-aligned row segment.  A and B are
// both K-contiguous ("NT"), which is the operand layout the MFMA wants.
//
// Design (CDNA4, wave64):
//   * block tile 128 x BN, K step 128 = one scale block; 8 waves (2 per SIMD)
//     as 2 (M) x 4 (N), each wave 64 x BN/4 built from 16x16x128 f8f6f4 MFMAs.
//     One MFMA covers exactly one scale block: its fresh fp32 partial is
//     rescaled by sA*sB and added to the fp32 accumulator with one VALU FMA
//     per element per block; MFMAs of the next n-subtile run meanwhile.
//   * operands stream global -> LDS directly (global_load_lds_dwordx4), three
//     stages deep: K blocks kb+1 and kb+2 are in flight while kb is
//     multiplied; one barrier per K block.  The LDS image of every 128-byte
//     row is XOR swizzled in 16-byte chunks (chunk c of row r is stored at
//     c ^ (r & 7)), and the four 16-lane groups of a fragment read take the
//     consecutive chunks g and g + 4: measured on gfx950, this pattern reads
//     at the full LDS rate while chunk pairs {2g, 2g+1} run at half rate from
//     bank conflicts.
//   * persistent blocks walk an expert-major tile list built on the device from
//     counts/offsets (no host sync); consecutive tiles share a weight tile and
//     are mapped to the same XCD so that weight tile is fetched into one L2.
//   * epilogues stage through LDS for coalesced 16-byte stores.
#include "mfma_common.hpp"

namespace moe {

constexpr int GBM = 128;
constexpr int GBK = 128;
constexpr int GTHREADS = 512;
constexpr int GWAVES = GTHREADS / 64;
constexpr int GMAXL = 1024;
constexpr int GMAXKB = 256;  // K <= 32768

struct GemmArgs {
    const uint8_t* a;
    const float* a_s;
    const uint8_t* b;
    const float* b_s;
    const int32_t* counts;
    const int32_t* offsets;
    int L;
    int64_t row_cap;
    int N;
    int K;
    const uint16_t* epi_in;
    void* out;
    float* out_s;
    void* out2;
    float* out2_s;
    void* out3;
    float* out3_s;
};
constexpr bool is_swiglu(int epi) {
    return epi == MOE_EPI_SWIGLU_Q8 || epi == MOE_EPI_SWIGLU_Q8_SAVE || epi == MOE_EPI_SWIGLU_F32;
}

template <int BN>
struct GemmSmem {
    static constexpr int A_BYTES = GBM * GBK;
    static constexpr int B_BYTES = BN * GBK;
    static constexpr int S_BYTES = GBM * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int NSTAGE = 3;
    static constexpr int TOTAL = NSTAGE * STAGE;
};

template <int BN, int EPI>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_fp8_kernel(GemmArgs g) {
    using SM = GemmSmem<BN>;
    constexpr int WN = BN / 4;        // wave tile columns
    constexpr int NI = WN / 16;       // n-subtiles per wave
    constexpr int ASEG = GBM / 8 / GWAVES;  // 1 KB A segments per wave
    constexpr int BSEG = BN / 8 / GWAVES;   // 1 KB B segments per wave
    constexpr int NLD = ASEG + BSEG + 1;    // DMA instructions per wave per stage
    static_assert(!is_swiglu(EPI) || BN == 256, "SwiGLU tiles pair 128 G with 128 U columns");

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    __shared__ int tile_base[GMAXL + 1];
    __shared__ int scan_tmp[GTHREADS];
    __shared__ float rowmax[4][GBM];
    __shared__ __attribute__((aligned(8))) float bscale[GMAXKB][2];  // this tile's B scales per K block

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave >> 2, wn = wave & 3;
    const int L = g.L, N = g.N, K = g.K;
    const int nkb = K / GBK;
    const int NT = N / BN;
    const int f = N / 2;  // SwiGLU: G = [0, f), U = [f, 2f)

    // ---- tile list: per-expert m-tiles of the (row_cap-clamped) padded segments
    {
        int loc[2];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid * 2 + i;
            int m = 0;
            if (e < L) {
                int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
                if (lo > g.row_cap) lo = g.row_cap;
                if (hi > g.row_cap) hi = g.row_cap;
                m = hi > lo ? (int)((hi - lo) / GBM) : 0;
            }
            loc[i] = m;
            sum += m;
        }
        scan_tmp[tid] = sum;
        __syncthreads();
        for (int off = 1; off < GTHREADS; off <<= 1) {
            int add = tid >= off ? scan_tmp[tid - off] : 0;
            __syncthreads();
            scan_tmp[tid] += add;
            __syncthreads();
        }
        int run = scan_tmp[tid] - sum;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid * 2 + i;
            if (e < L) tile_base[e] = run * NT;
            run += loc[i];
        }
        if (tid == 0) tile_base[L] = scan_tmp[GTHREADS - 1] * NT;
        __syncthreads();
    }
    const int total = tile_base[L];
    const int G = gridDim.x;  // a multiple of 8
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // per-lane LDS read offsets (stage-relative).  Lane l holds row l & 15 of a
    // fragment and K chunks g and g + 4 of the 128-byte block (g = l >> 4);
    // A and B use the same lane -> K mapping, so the MFMA sums the same
    // products.  row & 7 == lane & 7 for every fragment row, so the swizzled
    // chunk is fixed per lane.
    const int l15 = lane & 15, l7 = lane & 7, c0 = lane >> 4;
    const uint32_t a_rd0 = (wm * 64 + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t a_rd1 = (wm * 64 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t b_rd0 = SM::A_BYTES + (wn * WN + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * WN + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t s_rd = SM::A_BYTES + SM::B_BYTES + (wm * 64 + (lane >> 4) * 4) * 4;

    for (int t = lb; t < total; t += G) {
        int lo = 0, hi = L;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tile_base[mid] <= t) lo = mid; else hi = mid;
        }
        const int e = __builtin_amdgcn_readfirstlane(lo);
        const int tb0 = __builtin_amdgcn_readfirstlane(tile_base[e]);
        const int tb1 = __builtin_amdgcn_readfirstlane(tile_base[e + 1]);
        const int mt_e = (tb1 - tb0) / NT;
        const int local = t - tb0;
        const int nt = local / mt_e, mt = local - nt * mt_e;
        const int64_t row0 = (int64_t)g.offsets[e] + (int64_t)mt * GBM;
        const int64_t real_end = (int64_t)g.offsets[e] + g.counts[e];
        const int n0 = nt * BN;  // STORE: first output column; SwiGLU: nt*128 is the first h column

        const uint8_t* Ag = g.a + row0 * K;
        const float* Asg = g.a_s + row0 * nkb;
        const uint8_t* Bg = g.b + (int64_t)e * N * K;

        // B scale rows (128-column blocks) of this wave: for SwiGLU the G block
        // (n-subtiles 0, 1) and the U block (2, 3); for stores one block holds
        // all of the wave's columns.  They are staged in LDS for the tile so
        // the K loop reads them together with the operand fragments.
        const float* bs_base = g.b_s + (int64_t)e * (N / 128) * nkb;
        int blk0, blk1;
        if constexpr (is_swiglu(EPI)) {
            blk0 = nt;              // G columns
            blk1 = f / 128 + nt;    // U columns
        } else {
            blk0 = n0 / 128;        // columns [n0, n0 + 128)
            blk1 = blk0 + (BN > 128 ? 1 : 0);
        }
        for (int i = tid; i < 2 * nkb; i += GTHREADS) {
            const int kb = i >> 1, which = i & 1;
            bscale[kb][which] = bs_base[(int64_t)(which ? blk1 : blk0) * nkb + kb];
        }
        const uint32_t bs_rd = lds_addr(&bscale[0][0]);
        // STORE: waves wn = 0, 1 use block blk0, wn = 2, 3 block blk1
        const bool second_blk = !is_swiglu(EPI) && BN > 128 && wn >= 2;

        // DMA sources.  Segment q (1 KB) holds tile rows 8q .. 8q+7; lane l moves
        // LDS chunk (l & 7) of row 8q + l/8, i.e. global chunk (l & 7) ^ (row & 7)
        // (the XOR swizzle is its own inverse; rows 8 apart share it).
        const int ra = wave * (ASEG * 8) + (lane >> 3);
        const uint8_t* a_src = Ag + (int64_t)ra * K + (((lane & 7) ^ (ra & 7)) << 4);
        const int rb = wave * (BSEG * 8) + (lane >> 3);
        int brow0;
        if constexpr (is_swiglu(EPI)) {
            // LDS B rows in 32-row blocks: block 2w' holds G columns nt*128 +
            // 32w' + [0, 32), block 2w'+1 the U columns of the same h columns;
            // wave w fills block w
            brow0 = ((wave & 1) ? f : 0) + nt * 128 + (wave >> 1) * 32 + (lane >> 3);
        } else {
            brow0 = n0 + rb;
        }
        const uint8_t* b_src = Bg + (int64_t)brow0 * K + (((lane & 7) ^ (rb & 7)) << 4);
        const float* s_src = Asg + (int64_t)(wave * 16 + (lane & 15)) * nkb;
        const int64_t K8 = (int64_t)8 * K;

        auto issue = [&](int stage, int kb) {
            const uint32_t sA = sbase + (uint32_t)(stage * SM::STAGE);
            const uint32_t sB = sA + SM::A_BYTES;
            const uint32_t sS = sB + SM::B_BYTES;
            const int kofs = kb * GBK;
#pragma unroll
            for (int i = 0; i < ASEG; ++i) dma16(a_src + i * K8 + kofs, sA + (wave * ASEG + i) * 1024);
#pragma unroll
            for (int i = 0; i < BSEG; ++i) dma16(b_src + i * K8 + kofs, sB + (wave * BSEG + i) * 1024);
            if (lane < 16) dma4(s_src + kb, sS + wave * 64);  // 16 rows' A scales per wave
        };

        v4f acc[4][NI];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

        __syncthreads();  // the previous tile's epilogue is done with smem
        issue(0, 0);
        if (nkb > 1) issue(1, 1);
        for (int kb = 0; kb < nkb; ++kb) {
            if (kb + 1 < nkb) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();  // stage kb landed for all waves; stage kb-1 no longer read
            if (kb + 2 < nkb) issue((kb + 2) % 3, kb + 2);
            const uint32_t base = opaque(sbase + (uint32_t)((kb % 3) * SM::STAGE));
            const uint32_t bsa = opaque(bs_rd + kb * 8);

            u32x4 alo[4], ahi[4], sa4[4], blo[2], bhi[2];
            const v2u sbv = lds8<0>(bsa);
            blo[0] = lds16<0>(base + b_rd0);
            bhi[0] = lds16<0>(base + b_rd1);
            static_for<0, 4>([&](auto ic) {
                constexpr int mi = decltype(ic)::value;
                alo[mi] = lds16<mi * 2048>(base + a_rd0);
                ahi[mi] = lds16<mi * 2048>(base + a_rd1);
                sa4[mi] = lds16<mi * 64>(base + s_rd);
            });
            v8i af[4];
            v4f sc0[4], sc1[4];
            v4f pt[2][4];
            // element values go through plain integers: __builtin_bit_cast of an
            // ext_vector element lvalue reads element 0 with this compiler
            const uint32_t sbx = sbv.x, sby = sbv.y;
            const float sb0 = __uint_as_float(second_blk ? sby : sbx);
            const float sb1 = __uint_as_float(sby);
            const v8i bf0 = join8(blo[0], bhi[0]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                af[mi] = join8(alo[mi], ahi[mi]);
                const v4f sa = __builtin_bit_cast(v4f, sa4[mi]);
                sc0[mi] = sa * sb0;
                if constexpr (is_swiglu(EPI)) sc1[mi] = sa * sb1;
                pt[0][mi] = mfma16x16x128(af[mi], bf0);
            }
            // software pipeline over n-subtiles: the MFMAs of subtile ni run
            // while the rescale-accumulate of subtile ni-1 retires on the VALU
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
                    constexpr bool second = is_swiglu(EPI) && pn >= NI / 2;
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi) acc[mi][pn] += pt[pn & 1][mi] * (second ? sc1[mi] : sc0[mi]);
                }
            });
        }
        __syncthreads();  // every wave is done reading the operand stages

        // ---------------------------------------------------------- epilogues
        // lane's rows: wm*64 + mi*16 + (lane>>4)*4 + i ; columns within the
        // tile: wn*WN + ni*16 + (lane & 15)
        const int rbase = wm * 64 + (lane >> 4) * 4;
        const int cl = lane & 15;
        if constexpr (EPI == MOE_EPI_STORE_F32) {
            float* out = static_cast<float*>(g.out);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t r = row0 + rbase + mi * 16 + i;
                    if (r >= real_end) continue;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) out[r * N + n0 + wn * WN + ni * 16 + cl] = acc[mi][ni][i];
                }
        } else if constexpr (EPI == MOE_EPI_STORE_BF16) {
            constexpr int LDR = BN * 2 + 16;  // staged row stride (bytes)
            static_assert(GBM * LDR <= SM::TOTAL, "staging fits");
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rbase + mi * 16 + i;
                        const int c = wn * WN + ni * 16 + cl;
                        *reinterpret_cast<uint16_t*>(smem + r * LDR + c * 2) = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                    }
            __syncthreads();
            uint16_t* out = static_cast<uint16_t*>(g.out);
            constexpr int CPR = BN / 8;  // 16-byte chunks per row
            for (int idx = tid; idx < GBM * CPR; idx += GTHREADS) {
                const int r = idx / CPR, ch = idx - r * CPR;
                if (row0 + r >= real_end) continue;
                const uint4 v = *reinterpret_cast<const uint4*>(smem + r * LDR + ch * 16);
                *reinterpret_cast<uint4*>(out + (row0 + r) * N + n0 + ch * 8) = v;
            }
        } else if constexpr (is_swiglu(EPI)) {
            // n-subtiles 0, 1 are G and 2, 3 the U of the same h columns
            // hcol = wn*32 + ni*16 + cl within this tile's 128 h columns
            float h[4][2][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gv = acc[mi][ni][i], uv = acc[mi][ni + 2][i];
                        h[mi][ni][i] = gv / (1.0f + expf(-gv)) * uv;
                    }
            const int hcol0 = nt * 128;
            if constexpr (EPI == MOE_EPI_SWIGLU_F32) {
                float* out = static_cast<float*>(g.out);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t r = row0 + rbase + mi * 16 + i;
                        if (r >= real_end) continue;
#pragma unroll
                        for (int ni = 0; ni < 2; ++ni) out[r * f + hcol0 + wn * 32 + ni * 16 + cl] = h[mi][ni][i];
                    }
            } else {
                // per-row amax over this wave's 32 h columns, then across the 4 N waves
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float m = fmaxf(fabsf(h[mi][0][i]), fabsf(h[mi][1][i]));
                        m = group_max<16>(m);
                        if (cl == 0) rowmax[wn][rbase + mi * 16 + i] = m;
                    }
                __syncthreads();
                constexpr int LDQ = 128 + 16;  // byte tile row stride
                uint8_t* qt = smem;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rbase + mi * 16 + i;
                        const float am = fmaxf(fmaxf(rowmax[0][r], rowmax[1][r]), fmaxf(rowmax[2][r], rowmax[3][r]));
                        const TileScale ts = tile_scale(am);
                        if (cl == 0 && wn == 0 && row0 + r < real_end) g.out_s[(row0 + r) * (f / 128) + nt] = ts.s;
                        const int w2 = cvt_e4m3x2(h[mi][0][i] * ts.inv, h[mi][1][i] * ts.inv);
                        qt[r * LDQ + wn * 32 + cl] = (uint8_t)(w2 & 0xFF);
                        qt[r * LDQ + wn * 32 + 16 + cl] = (uint8_t)((w2 >> 8) & 0xFF);
                    }
                if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                    // G and U as bf16, staged after the byte tile
                    constexpr int LDG = 256 * 2 + 16;
                    uint8_t* gt = smem + GBM * LDQ;
                    static_assert(GBM * LDQ + GBM * LDG <= SM::TOTAL, "staging fits");
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = rbase + mi * 16 + i;
                                const int c = wn * 32 + ni * 16 + cl;
                                *reinterpret_cast<uint16_t*>(gt + r * LDG + c * 2) =
                                    (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                                *reinterpret_cast<uint16_t*>(gt + r * LDG + 256 + c * 2) =
                                    (uint16_t)f32_to_bf16(acc[mi][ni + 2][i]);
                            }
                }
                __syncthreads();
                uint8_t* out = static_cast<uint8_t*>(g.out);
                for (int idx = tid; idx < GBM * 8; idx += GTHREADS) {
                    const int r = idx >> 3, ch = idx & 7;
                    if (row0 + r >= real_end) continue;
                    const uint4 v = *reinterpret_cast<const uint4*>(qt + r * LDQ + ch * 16);
                    *reinterpret_cast<uint4*>(out + (row0 + r) * f + hcol0 + ch * 16) = v;
                }
                if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                    constexpr int LDG = 256 * 2 + 16;
                    const uint8_t* gt = smem + GBM * LDQ;
                    uint16_t* out2 = static_cast<uint16_t*>(g.out2);
                    for (int idx = tid; idx < GBM * 32; idx += GTHREADS) {
                        const int r = idx >> 5, ch = idx & 31;  // 16 chunks of G then 16 of U
                        if (row0 + r >= real_end) continue;
                        const uint4 v = *reinterpret_cast<const uint4*>(gt + r * LDG + ch * 16);
                        const int col = (ch < 16 ? 0 : f) + hcol0 + (ch & 15) * 8;
                        *reinterpret_cast<uint4*>(out2 + (row0 + r) * N + col) = v;
                    }
                }
            }
        }
        // the next tile's first __syncthreads protects smem reuse
    }
}

template <int BN, int EPI>
static int launch_gemm(const GemmArgs& a, hipStream_t stream) {
    const int ncu = num_cus();
    const int grid = (ncu + 7) / 8 * 8;  // one 512-thread block per CU (LDS bound), persistent
    gemm_fp8_kernel<BN, EPI><<<dim3(grid), dim3(GTHREADS), 0, stream>>>(a);
    MOE_LAUNCH_CHECK("gemm_fp8_kernel");
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_gemm_fp8(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                                    const int32_t* counts, const int32_t* offsets, int32_t L, int64_t row_cap,
                                    int32_t N, int32_t K, int32_t epilogue, const uint16_t* epi_in, void* out,
                                    float* out_s, void* out2, float* out2_s, void* out3, float* out3_s,
                                    hipStream_t stream) {
    MOE_REQUIRE(L >= 1 && L <= GMAXL, MOE_ERR_SHAPE, "grouped_gemm: L=%d outside [1, 1024]", L);
    MOE_REQUIRE(row_cap >= 0 && row_cap % GBM == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "grouped_gemm: row_cap=%lld must be a multiple of 128", (long long)row_cap);
    MOE_REQUIRE(N > 0 && N % 128 == 0 && K > 0 && K % 128 == 0 && K / 128 <= GMAXKB, MOE_ERR_SHAPE,
                "grouped_gemm: N=%d, K=%d must be multiples of 128 with K <= 32768", N, K);
    MOE_REQUIRE(epilogue >= MOE_EPI_STORE_BF16 && epilogue <= MOE_EPI_SWIGLU_F32, MOE_ERR_UNSUPPORTED,
                "grouped_gemm: epilogue %d not supported", epilogue);
    const bool swiglu = epilogue == MOE_EPI_SWIGLU_Q8 || epilogue == MOE_EPI_SWIGLU_Q8_SAVE ||
                        epilogue == MOE_EPI_SWIGLU_F32;
    MOE_REQUIRE(!swiglu || N % 256 == 0, MOE_ERR_SHAPE, "grouped_gemm: SwiGLU needs N = 2f with f %% 128 == 0");
    MOE_REQUIRE(a && a_s && b && b_s && counts && offsets && out, MOE_ERR_NULL, "grouped_gemm: NULL argument");
    MOE_REQUIRE(epilogue != MOE_EPI_SWIGLU_Q8 || out_s, MOE_ERR_NULL, "grouped_gemm: SWIGLU_Q8 needs out_s");
    MOE_REQUIRE(epilogue != MOE_EPI_SWIGLU_Q8_SAVE || (out_s && out2), MOE_ERR_NULL,
                "grouped_gemm: SWIGLU_Q8_SAVE needs out_s and out2");
    MOE_REQUIRE((row_cap / GBM) * (N / 128) < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "grouped_gemm: row_cap * N too large for the tile list");
    if (row_cap == 0) return MOE_OK;
    GemmArgs ga{a, a_s, b, b_s, counts, offsets, L, row_cap, N, K, epi_in, out, out_s, out2, out2_s, out3, out3_s};
    const bool wide = N % 256 == 0;
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            return wide ? launch_gemm<256, MOE_EPI_STORE_BF16>(ga, stream)
                        : launch_gemm<128, MOE_EPI_STORE_BF16>(ga, stream);
        case MOE_EPI_STORE_F32:
            return wide ? launch_gemm<256, MOE_EPI_STORE_F32>(ga, stream)
                        : launch_gemm<128, MOE_EPI_STORE_F32>(ga, stream);
        case MOE_EPI_SWIGLU_Q8:
            return launch_gemm<256, MOE_EPI_SWIGLU_Q8>(ga, stream);
        case MOE_EPI_SWIGLU_Q8_SAVE:
            return launch_gemm<256, MOE_EPI_SWIGLU_Q8_SAVE>(ga, stream);
        case MOE_EPI_SWIGLU_F32:
            return launch_gemm<256, MOE_EPI_SWIGLU_F32>(ga, stream);
    }
    return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm: epilogue %d", epilogue);
}
