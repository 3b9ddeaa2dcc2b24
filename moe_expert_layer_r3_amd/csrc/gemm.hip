// Block-scaled FP8 grouped GEMM on gfx950 MFMA ("RL at 1T scale", section "FP8
// Training": block-scaled FP8 trainer GEMMs in the DeepSeek-V3 style).
//
// C[r, n] = sum_c sA[r, c] * sB[n/128, c] * (A[r, 128c:128c+128] . B[n, 128c:128c+128])
// for the real rows r of each expert's 128-aligned row segment.  A and B are
// both K-contiguous ("NT"), which is the operand layout the MFMA wants.
//
// Design (CDNA4, wave64):
//   * block tile 128 x BN, K step 128 = one scale block; 4 waves as 2 x 2, each
//     wave 64 x BN/2 built from 16x16x128 f8f6f4 MFMAs: one MFMA covers exactly
//     one scale block, so its fresh fp32 result is rescaled by sA*sB and added
//     to the fp32 accumulator (one VALU FMA per accumulator per K block).
//   * operands stream global -> registers -> LDS, double buffered: the loads
//     of K block kb+1 are in flight while block kb is multiplied; the LDS
//     image of every 128-byte row is XOR swizzled in 16-byte chunks so the
//     fragment reads are bank-conflict free.
//   * persistent blocks walk an expert-major tile list built on the device from
//     counts/offsets (no host sync); consecutive tiles share a weight tile and
//     are mapped to the same XCD so that weight tile is fetched into one L2.
//   * epilogues stage through LDS for coalesced 16-byte stores.
#include "common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 128;
constexpr int GBK = 128;
constexpr int GTHREADS = 256;
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
    static constexpr int TOTAL = 2 * STAGE;
};

// Byte offset of (row r, 16-byte chunk c) in a 128-byte-row operand image.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// MFMA 16x16x128 operand fragment: lane l holds 32 K-bytes of row r, chunks
// 2*(l/16) and 2*(l/16)+1 of the 128-byte K block.  A and B use the same
// lane -> K mapping, so any fixed permutation of K inside the block leaves the
// dot products unchanged.
__device__ __forceinline__ v8i frag_read(const uint8_t* base, int r, int lane) {
    const int c0 = (lane >> 4) * 2;
    const u32x4 lo4 = *reinterpret_cast<const u32x4*>(base + swz(r, c0));
    const u32x4 hi4 = *reinterpret_cast<const u32x4*>(base + swz(r, c0 + 1));
    return v8i{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w, (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
}

template <int BN, int EPI>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_fp8_kernel(GemmArgs g) {
    using SM = GemmSmem<BN>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    __shared__ int tile_base[GMAXL + 1];
    __shared__ int scan_tmp[GTHREADS];
    __shared__ float bscale[2][GMAXKB];
    __shared__ float rowmax[2][GBM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int L = g.L, N = g.N, K = g.K;
    const int nkb = K / GBK;
    const int NT = N / BN;
    const int f = N / 2;  // SwiGLU: G = [0, f), U = [f, 2f)

    // ---- tile list: per-expert m-tiles of the (row_cap-clamped) padded segments
    {
        int loc[4];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
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
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            if (e < L) tile_base[e] = run * NT;
            run += loc[i];
        }
        if (tid == 0) tile_base[L] = scan_tmp[GTHREADS - 1] * NT;
        __syncthreads();
    }
    const int total = tile_base[L];
    const int G = gridDim.x;  // a multiple of 8
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    for (int t = lb; t < total; t += G) {
        int lo = 0, hi = L;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tile_base[mid] <= t) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int mt_e = (tile_base[e + 1] - tile_base[e]) / NT;
        const int local = t - tile_base[e];
        const int nt = local / mt_e, mt = local - nt * mt_e;
        const int64_t row0 = (int64_t)g.offsets[e] + (int64_t)mt * GBM;
        const int64_t real_end = (int64_t)g.offsets[e] + g.counts[e];
        const int n0 = nt * BN;  // STORE: first output column; SwiGLU: nt*128 is the h column

        const uint8_t* Ag = g.a + row0 * K;
        const float* Asg = g.a_s + row0 * nkb;
        const uint8_t* Bg = g.b + (int64_t)e * N * K;

        // B scales of the (at most two) 128-column blocks this tile touches
        {
            int blk0, blk1;
            if constexpr (is_swiglu(EPI)) {
                blk0 = nt;
                blk1 = f / 128 + nt;
            } else {
                blk0 = n0 / 128;
                blk1 = BN > 128 ? blk0 + 1 : blk0;
            }
            const float* bs = g.b_s + (int64_t)e * (N / 128) * nkb;
            for (int i = tid; i < 2 * nkb; i += GTHREADS) {
                const int which = i / nkb, kb = i - which * nkb;
                bscale[which][kb] = bs[(int64_t)(which ? blk1 : blk0) * nkb + kb];
            }
        }


        // Global -> register -> LDS staging.  Thread (wave, lane) moves 16-byte
        // chunk `lane` of each 1 KB LDS segment q it owns; the global address is
        // the inverse of the swizzle so the LDS image is the swizzled layout.
        constexpr int NBL = BN / 32;  // B segments per wave
        u32x4 ra[4], rb[NBL];
        float rs = 0.f;
        int64_t a_off[4], b_off[NBL];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = wave * 4 + i;
            const int r = q * 8 + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            a_off[i] = (int64_t)r * K + c * 16;
        }
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const int q = wave * NBL + i;
            const int rr = q * 8 + (lane >> 3);
            const int c = (lane & 7) ^ (rr & 7);
            int br;
            if constexpr (is_swiglu(EPI)) {
                const int blk = rr >> 6;
                br = ((blk & 1) ? f : 0) + nt * 128 + (blk >> 1) * 64 + (rr & 63);
            } else {
                br = n0 + rr;
            }
            b_off[i] = (int64_t)br * K + c * 16;
        }
        const float* s_src = Asg + (int64_t)(wave * 32 + (lane & 31)) * nkb;
#define MOE_GLOAD(kb_)                                                                               \
    do {                                                                                             \
        const int kofs_ = (kb_) * GBK;                                                               \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) ra[i] =                                        \
            *reinterpret_cast<const u32x4*>(Ag + a_off[i] + kofs_);                                  \
        _Pragma("unroll") for (int i = 0; i < NBL; ++i) rb[i] =                                      \
            *reinterpret_cast<const u32x4*>(Bg + b_off[i] + kofs_);                                  \
        if (lane < 32) rs = s_src[(kb_)];                                                            \
    } while (0)
#define MOE_LSTORE(stage_)                                                                           \
    do {                                                                                             \
        uint8_t* sA_ = smem + (stage_) * SM::STAGE;                                                  \
        uint8_t* sB_ = sA_ + SM::A_BYTES;                                                            \
        float* sS_ = reinterpret_cast<float*>(sB_ + SM::B_BYTES);                                    \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                \
            *reinterpret_cast<u32x4*>(sA_ + (wave * 4 + i) * 1024 + lane * 16) = ra[i];              \
        _Pragma("unroll") for (int i = 0; i < NBL; ++i)                                              \
            *reinterpret_cast<u32x4*>(sB_ + (wave * NBL + i) * 1024 + lane * 16) = rb[i];            \
        if (lane < 32) sS_[wave * 32 + lane] = rs;                                                   \
    } while (0)

        v4f acc[4][8];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = zero;

        __syncthreads();  // bscale visible; previous tile's epilogue done with smem
        MOE_GLOAD(0);
        MOE_LSTORE(0);
        __syncthreads();
        constexpr int NI = BN == 128 ? 4 : 8;  // n-subtiles per wave
        for (int kb = 0; kb < nkb; ++kb) {
            if (kb + 1 < nkb) MOE_GLOAD(kb + 1);
            const uint8_t* sA = smem + (kb & 1) * SM::STAGE;
            const uint8_t* sB = sA + SM::A_BYTES;
            const float* sS = reinterpret_cast<const float*>(sB + SM::B_BYTES);

            v8i af[4];
            v4f sc0[4], sc1[4];
            // STORE: the wave's BN/2 columns lie in one 128-column block of B
            const float sb0 = is_swiglu(EPI) ? bscale[0][kb] : bscale[(BN > 128 && wn) ? 1 : 0][kb];
            const float sb1 = bscale[1][kb];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                af[mi] = frag_read(sA, wm * 64 + mi * 16 + (lane & 15), lane);
                const float4 sa = *reinterpret_cast<const float4*>(sS + wm * 64 + mi * 16 + (lane >> 4) * 4);
                sc0[mi] = v4f{sa.x * sb0, sa.y * sb0, sa.z * sb0, sa.w * sb0};
                if constexpr (is_swiglu(EPI)) sc1[mi] = v4f{sa.x * sb1, sa.y * sb1, sa.z * sb1, sa.w * sb1};
            }
            // software pipeline: the MFMAs of n-subtile ni run while the
            // rescale-accumulate of n-subtile ni-1 retires on the VALU
            v4f pt[2][4];
            {
                const v8i bf = frag_read(sB, wn * (BN / 2) + (lane & 15), lane);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    pt[0][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf, zero, 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
            for (int ni = 1; ni <= NI; ++ni) {
                if (ni < NI) {
                    const v8i bf = frag_read(sB, wn * (BN / 2) + ni * 16 + (lane & 15), lane);
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
                        pt[ni & 1][mi] =
                            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf, zero, 0, 0, 0, 127, 0, 127);
                }
                const int pn = ni - 1;
                const bool second = is_swiglu(EPI) && pn >= 4;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) acc[mi][pn] += pt[pn & 1][mi] * (second ? sc1[mi] : sc0[mi]);
            }
            if (kb + 1 < nkb) MOE_LSTORE((kb + 1) & 1);
            __syncthreads();
        }

        // ---------------------------------------------------------- epilogues
        // lane's rows: wm*64 + mi*16 + (lane>>4)*4 + i ; column within the wave
        // tile: ni*16 + (lane & 15)
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
                    for (int ni = 0; ni < 8; ++ni) {
                        if (BN == 128 && ni >= 4) break;
                        out[r * N + n0 + wn * (BN / 2) + ni * 16 + cl] = acc[mi][ni][i];
                    }
                }
        } else if constexpr (EPI == MOE_EPI_STORE_BF16) {
            constexpr int LDR = BN * 2 + 16;  // staged row stride (bytes)
            static_assert(GBM * LDR <= SM::TOTAL, "staging fits");
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 8; ++ni) {
                    if (BN == 128 && ni >= 4) break;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = rbase + mi * 16 + i;
                        const int c = wn * (BN / 2) + ni * 16 + cl;
                        *reinterpret_cast<uint16_t*>(smem + r * LDR + c * 2) = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                    }
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
            // SwiGLU: n-subtile ni < 4 is G, ni + 4 is U of the same h column
            // hcol = wn*64 + ni*16 + cl within this tile's 128 h columns
            float h[4][4][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gv = acc[mi][ni][i], uv = acc[mi][ni + 4][i];
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
                        for (int ni = 0; ni < 4; ++ni) out[r * f + hcol0 + wn * 64 + ni * 16 + cl] = h[mi][ni][i];
                    }
            } else {
                // per-row amax over this wave's 64 h columns, then across the two N waves
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float m = 0.f;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) m = fmaxf(m, fabsf(h[mi][ni][i]));
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
                        const TileScale ts = tile_scale(fmaxf(rowmax[0][r], rowmax[1][r]));
                        if (cl == 0 && wn == 0 && row0 + r < real_end)
                            g.out_s[(row0 + r) * (f / 128) + nt] = ts.s;
#pragma unroll
                        for (int ni = 0; ni < 4; ni += 2) {
                            const int w2 = cvt_e4m3x2(h[mi][ni][i] * ts.inv, h[mi][ni + 1][i] * ts.inv);
                            qt[r * LDQ + wn * 64 + ni * 16 + cl] = (uint8_t)(w2 & 0xFF);
                            qt[r * LDQ + wn * 64 + (ni + 1) * 16 + cl] = (uint8_t)((w2 >> 8) & 0xFF);
                        }
                    }
                if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                    // G and U as bf16, staged after the byte tile
                    constexpr int LDG = 256 * 2 + 16;
                    uint8_t* gt = smem + GBM * LDQ;
                    static_assert(GBM * LDQ + GBM * LDG <= SM::TOTAL, "staging fits");
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = rbase + mi * 16 + i;
                                const int c = wn * 64 + ni * 16 + cl;
                                *reinterpret_cast<uint16_t*>(gt + r * LDG + c * 2) =
                                    (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                                *reinterpret_cast<uint16_t*>(gt + r * LDG + 256 + c * 2) =
                                    (uint16_t)f32_to_bf16(acc[mi][ni + 4][i]);
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
    int grid = ncu;  // one 256-thread block per CU (LDS bound), persistent
    grid = (grid + 7) / 8 * 8;
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
    (void)epi_in;
    (void)out2_s;
    (void)out3;
    (void)out3_s;
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

extern "C" int moe_grouped_gemm_fp8_wgrad(const uint8_t* aT, const float* aT_s, const uint8_t* bT,
                                          const float* bT_s, const int32_t* offsets, int32_t L, int64_t row_cap,
                                          int32_t M, int32_t N, uint16_t* dW, hipStream_t stream) {
    (void)aT; (void)aT_s; (void)bT; (void)bT_s; (void)offsets; (void)L; (void)row_cap; (void)M; (void)N;
    (void)dW; (void)stream;
    return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm_wgrad: not available in this build");
}
