// Thin last m-tiles of the SwiGLU grouped GEMM (MOE_GEMM_THIN_SPLIT): the
// K-split product and its epilogue.  The product is the block-scaled one of
// gemm.hip ("RL at 1T scale", section "FP8 Training"); only the order of the
// fp32 block sums differs.
//
// Work item (thin expert j, n-tile nt, K run s): the expert's last rows (at
// most 32, two 16-row subtiles) times the n-tile's 256 weight rows (128 of G
// and the matching 128 of U) over K blocks [4s, 4s + 4).  Four waves, one per
// 64 weight rows; fragments come straight from global memory into registers
// (the next K block's loads are issued before the current one multiplies),
// and each 16x16x128 MFMA's fresh partial is rescaled by sA * sB into the
// fp32 accumulator.  The partial tile [32 rows][256 columns] goes to the
// workspace slot of (expert, n-tile, run).
//
// Epilogue item (thin expert, n-tile): thread t owns row t / 8 and h columns
// 16 (t % 8) .. +15; it sums the K runs in order, forms h = silu(G) * U with the
// main product's arithmetic, and quantises the row's 128-column tile (an
// 8-lane maximum), or writes fp32 h for the inspection epilogue.
#include "mfma_common.hpp"
#include "gemm_thin.hpp"

namespace moe {

constexpr int TTHREADS = 256;
constexpr int TMAXL = 1024;

struct ThinArgs {
    const uint8_t* a;
    const float* a_s;
    const uint8_t* b;
    const float* b_s;
    const int32_t* counts;
    const int32_t* offsets;
    int L;
    int64_t row_cap;
    int N;  // 2f
    int K;
    float* ws;  // [L][N/256][splits][32][256] fp32 partials
    int G;      // workgroups of the main product (thin_split_active)
    void* out;
    float* out_s;
    uint16_t* out2;
};

// The experts with a thin last m-tile, in expert order, into list[]; returns
// their count (every thread), or 0 when the main product keeps those tiles
// (thin_split_active over all experts' m-tiles, as the product decides it).
// Wave 0 scans 64 experts per ballot.
__device__ __forceinline__ int thin_list(const ThinArgs& g, int* list, int* nlist) {
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        int n = 0, mt = 0;
        for (int c = 0; c < g.L; c += 64) {
            const int e = c + lane;
            const int64_t rows = e < g.L ? thin_seg_rows(g.counts, g.offsets, e, g.row_cap) : 0;
            const bool thin = thin_rows_of(rows) > 0;
            int m = (int)((rows + THIN_WBM - 1) / THIN_WBM);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m += __shfl_xor(m, o);
            mt += m;
            const uint64_t b = __ballot(thin);
            const int below =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (thin) list[n + below] = e;
            n += __popcll(b);
        }
        if (lane == 0) *nlist = thin_split_active(mt, n, g.N / 256, g.G) ? n : 0;
    }
    __syncthreads();
    return *nlist;
}

// first row of the expert's thin tile, its row count and the end of the rows
// its operand may be read from
struct ThinTile {
    int64_t r0;
    int rows;
    int64_t lim;
};
__device__ __forceinline__ ThinTile thin_tile(const ThinArgs& g, int e) {
    const int64_t rows = thin_seg_rows(g.counts, g.offsets, e, g.row_cap);
    ThinTile t;
    t.rows = thin_rows_of(rows);
    t.r0 = (int64_t)g.offsets[e] + (rows - t.rows);
    int64_t lim = g.offsets[e + 1];
    if (lim > g.row_cap) lim = g.row_cap;
    t.lim = lim;
    return t;
}

__global__ __launch_bounds__(TTHREADS) void gemm_thin_part_kernel(ThinArgs g) {
    __shared__ int list[TMAXL];
    __shared__ int nlist;
    const int nthin = thin_list(g, list, &nlist);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NT = g.N / 256, f = g.N / 2, nkb = g.K / 128, S = thin_splits(g.K);
    const int items = nthin * NT * S;
    const int l15 = lane & 15, grp = lane >> 4;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int j = it / (NT * S), rem = it - j * (NT * S);
        const int nt = rem / S, s = rem - nt * S;
        const int e = list[j];
        const ThinTile tt = thin_tile(g, e);
        const int kb0 = s * THIN_KB, kb1 = min(nkb, kb0 + THIN_KB);
        // this wave's 64 weight rows: G rows for waves 0-1, U rows for 2-3
        const int wrow = ((wave >> 1) ? f : 0) + nt * 128 + 64 * (wave & 1);
        const float* sb_row = g.b_s + ((int64_t)e * (g.N / 128) + wrow / 128) * nkb;
        // A rows of the lane (two 16-row subtiles), clamped inside the segment
        int64_t ar[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            int64_t r = tt.r0 + mi * 16 + l15;
            ar[mi] = r < tt.lim ? r : tt.lim - 1;
        }
        const uint8_t* ap[2] = {g.a + ar[0] * g.K + 32 * grp, g.a + ar[1] * g.K + 32 * grp};
        const uint8_t* bp = g.b + ((int64_t)e * g.N + wrow + l15) * g.K + 32 * grp;
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        v4f acc[2][4];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = zero;
        // fragments of K block kb: lane group grp holds its bytes [32 grp, 32 grp + 32)
        // for A and B alike (the product pairs equal K positions)
        auto fetch = [&](int kb, v8i (&af)[2], v8i (&bf)[4], float (&sa)[2], float& sbv) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(ap[mi] + (int64_t)kb * 128);
                const u32x4 y = *reinterpret_cast<const u32x4*>(ap[mi] + (int64_t)kb * 128 + 16);
                af[mi] = join8(x, y);
                sa[mi] = g.a_s[(int64_t)kb * g.row_cap + ar[mi]];
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const uint8_t* q = bp + (int64_t)ni * 16 * g.K + (int64_t)kb * 128;
                bf[ni] = join8(*reinterpret_cast<const u32x4*>(q), *reinterpret_cast<const u32x4*>(q + 16));
            }
            sbv = sb_row[kb];
        };
        v8i af[2], bf[4], af2[2], bf2[4];
        float sa[2], sa2[2], sbv = 0.f, sbv2 = 0.f;
        fetch(kb0, af, bf, sa, sbv);
        for (int kb = kb0; kb < kb1; ++kb) {
            if (kb + 1 < kb1) fetch(kb + 1, af2, bf2, sa2, sbv2);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const float sc = sa[mi] * sbv;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] += mfma16x16x128(bf[ni], af[mi]) * sc;
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                af[mi] = af2[mi];
                sa[mi] = sa2[mi];
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bf[ni] = bf2[ni];
            sbv = sbv2;
        }
        // partial [m][c]: lane holds rows mi*16 + l15, columns 64 wave + 16 ni + 4 grp .. +3
        float* p = g.ws + (((int64_t)e * NT + nt) * S + s) * (32 * 256);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                *reinterpret_cast<v4f*>(p + (mi * 16 + l15) * 256 + 64 * wave + 16 * ni + 4 * grp) = acc[mi][ni];
    }
}

template <int EPI, bool P2>
__global__ __launch_bounds__(TTHREADS) void gemm_thin_epi_kernel(ThinArgs g) {
    __shared__ int list[TMAXL];
    __shared__ int nlist;
    const int nthin = thin_list(g, list, &nlist);
    const int tid = threadIdx.x;
    const int NT = g.N / 256, f = g.N / 2, S = thin_splits(g.K);
    const int m = tid >> 3, c0 = (tid & 7) * 16;
    for (int it = blockIdx.x; it < nthin * NT; it += gridDim.x) {
        const int j = it / NT, nt = it - j * NT;
        const int e = list[j];
        const ThinTile tt = thin_tile(g, e);
        // the 8 threads of a row share m, so a row's lanes leave together
        if (m >= tt.rows) continue;
        float G[16], U[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) G[i] = U[i] = 0.f;
        const float* p = g.ws + ((int64_t)e * NT + nt) * S * (32 * 256) + m * 256 + c0;
        for (int s = 0; s < S; ++s) {
            const float* q = p + (int64_t)s * (32 * 256);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const v4f x = *reinterpret_cast<const v4f*>(q + 4 * v);
                const v4f y = *reinterpret_cast<const v4f*>(q + 128 + 4 * v);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    G[4 * v + c] += x[c];
                    U[4 * v + c] += y[c];
                }
            }
        }
        const int64_t r = tt.r0 + m;
        const int64_t hc = (int64_t)nt * 128 + c0;
        float h[16];
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            h[i] = silu(G[i]) * U[i];
            am = fmaxf(am, fabsf(h[i]));
        }
        if constexpr (EPI == MOE_EPI_SWIGLU_F32) {
            float* out = static_cast<float*>(g.out) + r * f + hc;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *reinterpret_cast<v4f*>(out + 4 * v) = v4f{h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]};
        } else {
            am = group_max<8>(am);
            const TileScale ts = tile_scale_t<P2>(am);
            u32x4 z;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                z[v] = cvt_e4m3x4(h[4 * v] * ts.inv, h[4 * v + 1] * ts.inv, h[4 * v + 2] * ts.inv,
                                  h[4 * v + 3] * ts.inv);
            *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(g.out) + r * f + hc) = z;
            if ((tid & 7) == 0) g.out_s[(int64_t)nt * g.row_cap + r] = ts.s;
            if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                u32x4 gb[2], ub[2];
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    gb[v >> 2][v & 3] = pack_bf16x2(G[2 * v], G[2 * v + 1]);
                    ub[v >> 2][v & 3] = pack_bf16x2(U[2 * v], U[2 * v + 1]);
                }
                uint16_t* o2 = g.out2 + r * g.N + hc;
                *reinterpret_cast<u32x4*>(o2) = gb[0];
                *reinterpret_cast<u32x4*>(o2 + 8) = gb[1];
                *reinterpret_cast<u32x4*>(o2 + f) = ub[0];
                *reinterpret_cast<u32x4*>(o2 + f + 8) = ub[1];
            }
        }
    }
}

}  // namespace moe

using namespace moe;

size_t moe_thin_workspace_bytes(int32_t L, int32_t N, int32_t K) {
    return (size_t)L * (size_t)(N / 256) * (size_t)thin_splits(K) * 32 * 256 * sizeof(float);
}

int moe_thin_launch(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s, const int32_t* counts,
                    const int32_t* offsets, int32_t L, int64_t row_cap, int32_t N, int32_t K, int32_t epilogue,
                    bool p2, float* ws, void* out, float* out_s, void* out2, hipStream_t stream) {
    // (the main product's grid: one workgroup per CU, a multiple of 8)
    const int grid = (num_cus() + 7) / 8 * 8;
    ThinArgs t{a, a_s, b, b_s, counts, offsets, L, row_cap, N, K, ws, grid, out, out_s,
               static_cast<uint16_t*>(out2)};
    gemm_thin_part_kernel<<<dim3(grid), dim3(TTHREADS), 0, stream>>>(t);
    MOE_LAUNCH_CHECK("gemm_thin_part_kernel");
    // (an epilogue item is one (expert, n-tile): a quarter of the grid covers
    // four thin experts of 16 n-tiles in one pass and leaves fast when none is)
    auto go = [&](auto kern) { kern<<<dim3(grid / 4), dim3(TTHREADS), 0, stream>>>(t); };
    switch (epilogue) {
        case MOE_EPI_SWIGLU_Q8:
            p2 ? go(gemm_thin_epi_kernel<MOE_EPI_SWIGLU_Q8, true>) : go(gemm_thin_epi_kernel<MOE_EPI_SWIGLU_Q8, false>);
            break;
        case MOE_EPI_SWIGLU_Q8_SAVE:
            p2 ? go(gemm_thin_epi_kernel<MOE_EPI_SWIGLU_Q8_SAVE, true>)
               : go(gemm_thin_epi_kernel<MOE_EPI_SWIGLU_Q8_SAVE, false>);
            break;
        case MOE_EPI_SWIGLU_F32:
            go(gemm_thin_epi_kernel<MOE_EPI_SWIGLU_F32, false>);
            break;
        default:
            return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm: thin split with epilogue %d", epilogue);
    }
    MOE_LAUNCH_CHECK("gemm_thin_epi_kernel");
    return MOE_OK;
}
