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
//     multiplied.  The LDS image of every 128-byte
//     row is XOR swizzled in 16-byte chunks (chunk c of row r is stored at
//     c ^ (r & 7)), and the four 16-lane groups of a fragment read take the
//     consecutive chunks g and g + 4: measured on gfx950, this pattern reads
//     at the full LDS rate while chunk pairs {2g, 2g+1} run at half rate from
//     bank conflicts.
//   * persistent blocks walk an expert-major tile list built on the device from
//     counts/offsets (no host sync); consecutive tiles share a weight tile and
//     are mapped to the same XCD so that weight tile is fetched into one L2.
//   * tiles that run side by side on an XCD and share an operand (the two
//     m-tiles of one weight tile, the n-tiles of one A tile) start their K loop
//     at different K blocks (a rotation of 2 per odd m-tile and 2 per n-tile
//     modulo 4): a neighbour's request for a line then finds it already in L2
//     instead of waiting on the same miss while holding a request slot
//     (measured: GEMM1 at 256 rows per expert 346 -> 313 us).  Only the order
//     of the fp32 block sums changes.
//   * epilogues write straight from registers.
//   * power-of-two scales (P2): every scale is 2^e, so sA*sB needs no fp32
//     multiply: the MFMA takes the two E8M0 exponents (one per operand row)
//     and accumulates the scaled block product into the fp32 accumulator
//     itself.  No partial waits for a VALU rescale, and the ring of raw
//     partials is gone.
//   * N % 256 == 0 runs the 256 x 256 variant of this product further below
//     (gemm_wide_kernel) unless the caller asks for this 128 x 256 one.
//   * MXFP4 weights (WF4, with P2 activations): B rows are 64 bytes per K step
//     (E2M1, two per byte) with one E8M0 scale per 32 values; a lane's B
//     fragment is the 16 bytes of K block lane/16 and its scale byte, and the
//     MFMA runs in the mixed fp4 x fp8 form.  Half the weight bytes per step.
#include "mfma_common.hpp"
#include "gemm_thin.hpp"

namespace moe {

constexpr int GBM = 128;
constexpr int GBK = 128;
constexpr int GTHREADS = 512;
constexpr int GWAVES = GTHREADS / 64;
constexpr int GMAXL = 1024;
constexpr int GMAXKB = 256;  // K <= 32768
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
#endif
constexpr int GROUP_M = MOE_GEMM_GROUP_M;  // m-tiles per L2 super-tile

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
    int thin;  // 1: thin last m-tiles are left to the K-split launches (gemm_thin.hip)
};
constexpr bool is_swiglu(int epi) {
    return epi == MOE_EPI_SWIGLU_Q8 || epi == MOE_EPI_SWIGLU_Q8_SAVE || epi == MOE_EPI_SWIGLU_F32;
}

template <int BN, bool WF4>
struct GemmSmem {
    static constexpr int A_BYTES = GBM * GBK;
    static constexpr int B_BYTES = BN * (WF4 ? GBK / 2 : GBK);
    static constexpr int S_BYTES = GBM * 4;
    static constexpr int BS_BYTES = WF4 ? BN * 4 : 0;  // E8M0 weight scales: 4 per row per K step
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + BS_BYTES;
    // three stages: the DMA runs two K steps ahead.  (A fourth stage fits
    // with fp4 weights and was measured: no gain, the stream is bound by
    // line requests per CU, not by latency.)
    static constexpr int NSTAGE = 3;
    static constexpr int TOTAL = NSTAGE * STAGE;
};

template <int BN, int EPI, bool P2, bool WF4>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_fp8_kernel(GemmArgs g) {
    using SM = GemmSmem<BN, WF4>;
    constexpr int WN = BN / 4;        // wave tile columns
    constexpr int NI = WN / 16;       // n-subtiles per wave
    constexpr int ASEG = GBM / 8 / GWAVES;  // 1 KB A segments per wave
    constexpr int BSEG = SM::B_BYTES / 1024 / GWAVES;  // 1 KB B segments per wave
    constexpr int BROWS = BN / GWAVES;      // B rows each wave loads (8 per fp8 segment, 16 per fp4 one)
    constexpr int NLD = ASEG + BSEG + 1 + (WF4 ? 1 : 0);  // DMA instructions per wave per stage
    static_assert(!WF4 || P2, "MXFP4 weights take the hardware-scale path");
    // Waiting for stage kb allows NLD younger loads (stage kb+1's DMA).  The
    // previous epilogue's global stores may also be outstanding; loads
    // complete in order, so a count of NLD still implies stage kb landed.
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
    // fp4 B rows are 64 bytes: 4 chunks, chunk c of row r stored at c ^ sw4(r)
    // with sw4(r) = ((r >> 1) ^ (r >> 3)) & 3, which keeps the 16 rows of a
    // fragment read on distinct banks; lane group g reads chunk g (K values
    // [32g, 32g + 32)), the natural partner of the A chunks g and g + 4
    const int sw4 = ((l15 >> 1) ^ (l15 >> 3)) & 3;
    const uint32_t b_rd0 = WF4 ? SM::A_BYTES + (wn * WN + l15) * 64 + ((c0 ^ sw4) << 4)
                               : SM::A_BYTES + (wn * WN + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * WN + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    // fp4 weight scales: 4 bytes per LDS B row (its four 32-blocks of the step)
    const uint32_t bq_rd = SM::A_BYTES + SM::B_BYTES + SM::S_BYTES + (wn * WN + l15) * 4 + c0;
    // A scales of a stage: 128 floats stored so that the 16 bytes at slot
    // wm*64 + 4*l15 hold the scales of rows wm*64 + mi*16 + l15, mi = 0..3 (the
    // rows of this lane's outputs), see the scale DMA below
    const uint32_t s_rd = SM::A_BYTES + SM::B_BYTES + (wm * 64 + l15 * 4) * 4;
    // the same offsets per stage, as full LDS addresses: with the stage a
    // compile-time constant in the (3x unrolled) K loop, every fragment read is
    // one ds_read with an immediate offset and no address arithmetic
    constexpr int NS = SM::NSTAGE;
    uint32_t rA0[NS], rA1[NS], rB0[NS], rB1[NS], rS[NS], rBS[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const uint32_t b = sbase + (uint32_t)(st * SM::STAGE);
        rA0[st] = b + a_rd0;
        rA1[st] = b + a_rd1;
        rB0[st] = b + b_rd0;
        rB1[st] = b + b_rd1;
        rBS[st] = b + bq_rd;
        rS[st] = b + s_rd;
    }

    // ---- per-tile parameters (all wave-uniform)
    struct Tile {
        int64_t row0, real_end;        // first row of the tile, end of the expert's real rows
        int nt, n0;                    // n-tile and its first output column (SwiGLU: first h column is nt*128)
        const uint8_t* a_base;         // this wave's first A row, K block 0
        const uint8_t* b_base;         // this wave's first B row, K block 0
        const uint8_t* bsm;            // fp4: this wave's first B row's E8M0 scales, K block 0
        const float* s_base;           // the tile's A scales
        const float* bs_lo;            // B scales of this wave's column blocks, K block 0
        const float* bs_hi;
        int rot;                       // first K block of the tile's loop (rotated order)
    };
    auto tile_at = [&](int t) {
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
        // super-tiles of up to GROUP_M m-tiles x all n-tiles, m fastest inside:
        // the 32 consecutive tiles an XCD runs at a time share few A and B tiles
        const int grp = local / (GROUP_M * NT);
        const int gm = min(GROUP_M, mt_e - grp * GROUP_M);
        const int in = local - grp * GROUP_M * NT;
        const int nt = in / gm, mt = grp * GROUP_M + (in - (in / gm) * gm);
        Tile ti;
        ti.row0 = (int64_t)g.offsets[e] + (int64_t)mt * GBM;
        ti.real_end = (int64_t)g.offsets[e] + g.counts[e];
        ti.nt = nt;
        ti.n0 = nt * BN;
        ti.a_base = g.a + (ti.row0 + wave * ASEG * 8) * K;
        int brow_w;  // first B row of this wave's DMA segments
        if constexpr (is_swiglu(EPI)) {
            // LDS B rows in 32-row blocks: block 2w' holds G columns nt*128 +
            // 32w' + [0, 32), block 2w'+1 the U columns of the same h columns;
            // wave w fills block w
            brow_w = ((wave & 1) ? f : 0) + nt * 128 + (wave >> 1) * 32;
        } else {
            brow_w = ti.n0 + wave * BROWS;
        }
        // fp4 codes are K-block-major [L, K/128, N, 64]: the wave's rows of one K
        // step are contiguous
        ti.b_base = WF4 ? g.b + ((int64_t)e * nkb * N + brow_w) * 64 : g.b + ((int64_t)e * N + brow_w) * K;
        ti.bsm = reinterpret_cast<const uint8_t*>(g.b_s) + ((int64_t)e * nkb * N + brow_w) * 4;
        ti.s_base = g.a_s + ti.row0;  // K-block-major: block kb's scales at kb * row_cap
        // B scale rows (128-column blocks): for SwiGLU the G block (n-subtiles
        // 0, 1) and the U block (2, 3); for stores waves wn = 0, 1 use the first
        // block of the tile and wn = 2, 3 the second
        const float* bsx = g.b_s + (int64_t)e * (N / 128) * nkb;
        int blk0, blk1;
        if constexpr (is_swiglu(EPI)) {
            blk0 = nt;
            blk1 = f / 128 + nt;
        } else {
            blk0 = ti.n0 / 128;
            blk1 = blk0 + (BN > 128 ? 1 : 0);
        }
        ti.bs_lo = bsx + (int64_t)blk0 * nkb;
        ti.bs_hi = bsx + (int64_t)blk1 * nkb;
        ti.rot = ((mt & 1) * 2 + (nt & 3) * 2) % nkb;
        return ti;
    };
    // B scales of a tile's two column blocks for every K block, staged in LDS
    // (read by the K loop together with the operand fragments)
    auto stage_bscale = [&](const Tile& ti) {
        if constexpr (WF4) return;  // per-row scales travel with the operand stages
        for (int i = tid; i < 2 * nkb; i += GTHREADS) {
            const int kb = i >> 1, which = i & 1;
            bscale[kb][which] = (which ? ti.bs_hi : ti.bs_lo)[kb];
        }
    };
    const uint32_t bs_rd = lds_addr(&bscale[0][0]);
    const bool second_blk = !is_swiglu(EPI) && BN > 128 && wn >= 2;

    // DMA lane offsets.  Segment q (1 KB) holds tile rows 8q .. 8q+7; lane l
    // moves LDS chunk (l & 7) of row 8q + l/8, i.e. global chunk (l & 7) ^ (row
    // & 7) (the XOR swizzle is its own inverse; rows 8 apart share it).  Every
    // source is a wave-uniform base (SGPRs) plus a 32-bit per-lane offset.
    const int lr = lane >> 3;  // row within a segment; every segment starts at a multiple of 8
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ lr) << 4);
    uint32_t a_off[ASEG], b_off[BSEG];
#pragma unroll
    for (int i = 0; i < ASEG; ++i) a_off[i] = (uint32_t)((8 * i + lr) * K) + chunk;
#pragma unroll
    for (int i = 0; i < BSEG; ++i) b_off[i] = (uint32_t)((8 * i + lr) * K) + chunk;
    if constexpr (WF4) {
        // fp4 segment: 16 rows of 64 bytes; lane l moves LDS chunk (l & 3) of
        // row l/4, i.e. global chunk (l & 3) ^ sw4(row) (segments start at
        // multiples of 16 rows, so the row within the segment sets the swizzle)
        const int r4 = lane >> 2;
        const uint32_t ch4 = (uint32_t)(((lane & 3) ^ (((r4 >> 1) ^ (r4 >> 3)) & 3)) << 4);
#pragma unroll
        for (int i = 0; i < BSEG; ++i) b_off[i] = (uint32_t)((16 * i + r4) * 64) + ch4;
    }
    const uint32_t bs_off = (uint32_t)(lane * 4);  // fp4 scales: lane l < BROWS fetches row l's 4 bytes
    // A scales (stored K-block-major, so a block's 128 row scales are 512
    // contiguous bytes): lane l < 16 of wave w fills scale slot w*16 + l, i.e.
    // row (w/4)*64 + (l%4)*16 + (w%4)*4 + l/4 (the layout the fragment reads
    // expect); one wave's 16 rows lie within 256 bytes
    const uint32_t s_off = (uint32_t)(((wave >> 2) * 64 + (lane & 3) * 16 + (wave & 3) * 4 + ((lane & 15) >> 2)) * 4);

    auto issue = [&](auto stage_c, int kb, const Tile& ti) {
        constexpr int stage = decltype(stage_c)::value;
        const uint32_t sA = sbase + (uint32_t)(stage * SM::STAGE);
        const uint32_t sB = sA + SM::A_BYTES;
        const uint32_t sS = sB + SM::B_BYTES;
        int kr = kb + ti.rot;  // K block in memory order
        if (kr >= nkb) kr -= nkb;
        const int kofs = kr * GBK;
#pragma unroll
        for (int i = 0; i < ASEG; ++i) dma16s(ti.a_base + kofs, a_off[i], sA + (wave * ASEG + i) * 1024);
        const int64_t kofs_b = WF4 ? (int64_t)kr * N * 64 : kofs;
#pragma unroll
        for (int i = 0; i < BSEG; ++i) dma16s(ti.b_base + kofs_b, b_off[i], sB + (wave * BSEG + i) * 1024);
        if constexpr (WF4) {
            if (lane < BROWS) dma4s(ti.bsm + (int64_t)kr * N * 4, bs_off, sS + SM::S_BYTES + wave * BROWS * 4);
        }
        if (lane < 16) dma4s(ti.s_base + (int64_t)kr * g.row_cap, s_off, sS + wave * 64);  // 16 rows' A scales
    };
    // barrier for LDS data only (s_waitcnt lgkmcnt(0) + s_barrier): unlike
    // __syncthreads it does not wait for the next tile's operand DMA in flight
    auto lds_barrier = [&]() {
        wait_lgkm0();
        phase_barrier();
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    // the first NS - 1 stages of a tile (all but one of the ring)
    auto prologue = [&](const Tile& ti) {
        static_for<0, NS - 1>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if (i < nkb) issue(std::integral_constant<int, i>{}, i, ti);
        });
    };
    // wait until stage kb has landed: the stages after it that are already
    // issued (up to NS - 2 of them) may stay in flight
    auto wait_stage = [&](int kb) {
        if constexpr (NS == 4) {
            if (kb + 2 < nkb) wait_vmcnt<2 * NLD>();
            else if (kb + 1 < nkb) wait_vmcnt<NLD>();
            else wait_vmcnt<0>();
        } else {
            if (kb + 1 < nkb) wait_vmcnt<NLD>(); else wait_vmcnt<0>();
        }
    };
    int t = lb;
    Tile cur;
    if (t < total) {
        cur = tile_at(t);
        stage_bscale(cur);
        lds_barrier();
        prologue(cur);
    }
    for (; t < total; t += G) {
        v4f acc[4][NI];
        v8i af[4], bfr[NI];   // fragments of one K block
        float sc0[4], sc1[4]; // sA * sB of that block per m-subtile (sc1: the U half of a SwiGLU tile)
        v4f ring[4];          // raw MFMA partials awaiting their rescale (4 in flight)
        int ea[4], eb0 = 127, eb1 = 127;  // P2: E8M0 codes of sA per m-subtile and of sB
        int eb4[NI];                      // WF4: E8M0 code of this lane's B row and K block per n-subtile
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;
            ring[mi] = zero4;
            sc0[mi] = sc1[mi] = 0.f;
        }

        // rescale-accumulate of the last n-subtile's partials, left in the ring
        // by the previous compute
        auto flush = [&]() {
            if constexpr (P2) return;
            constexpr bool second = is_swiglu(EPI) && (NI - 1) >= NI / 2;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi][NI - 1] += ring[mi] * (second ? sc1[mi] : sc0[mi]);
        };
        // operand fragments and scales of K block kb from its LDS stage (the
        // stage was published by the preceding barrier); the pending rescale
        // of the previous block runs while the reads are in flight
        auto load = [&](auto stage_c, int kb) {
            constexpr int st = decltype(stage_c)::value;
            // opaque: the reads may not be hoisted above the barrier that
            // published the stage
            const uint32_t pa0 = opaque(rA0[st]), pa1 = opaque(rA1[st]);
            const uint32_t pb0 = opaque(rB0[st]), pb1 = opaque(rB1[st]), ps = opaque(rS[st]);
            int kr = kb + cur.rot;
            if (kr >= nkb) kr -= nkb;
            const uint32_t bsa = opaque(bs_rd + kr * 8);
            const v2u sbv = lds8<0>(bsa);
            const u32x4 sa4 = lds16<0>(ps);
            static_for<0, 4>([&](auto ic) {
                constexpr int mi = decltype(ic)::value;
                af[mi] = join8(lds16<mi * 2048>(pa0), lds16<mi * 2048>(pa1));
            });
            if constexpr (WF4) {
                const uint32_t pbs = opaque(rBS[st]);
                const u32x4 z4 = {0u, 0u, 0u, 0u};
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    bfr[ni] = join8(lds16<ni * 1024>(pb0), z4);
                    eb4[ni] = (int)lds1<ni * 64>(pbs);
                });
            } else {
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    bfr[ni] = join8(lds16<ni * 2048>(pb0), lds16<ni * 2048>(pb1));
                });
            }
            flush();
            // element values go through plain integers: __builtin_bit_cast of an
            // ext_vector element lvalue reads element 0 with this compiler
            const uint32_t sbx = sbv.x, sby = sbv.y;
            const uint32_t sav[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
            if constexpr (P2) {
                // positive powers of two: the E8M0 code is the exponent field
                eb0 = (int)((second_blk ? sby : sbx) >> 23);
                eb1 = (int)(sby >> 23);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) ea[mi] = (int)(sav[mi] >> 23);
            } else {
                const float sb0 = __uint_as_float(second_blk ? sby : sbx);
                const float sb1 = __uint_as_float(sby);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const float sa = __uint_as_float(sav[mi]);
                    sc0[mi] = sa * sb0;
                    if constexpr (is_swiglu(EPI)) sc1[mi] = sa * sb1;
                }
            }
            wait_lgkm0();  // this wave's reads of the stage are complete before the next barrier
        };
        // the 4*NI MFMAs of the loaded block in (n-subtile, m-subtile) order,
        // weights as the first operand so that a lane's four outputs are four
        // consecutive columns of one row; MFMA j reuses the ring slot of MFMA
        // j-4 right after that partial's rescale, so four MFMAs are in flight
        // between a result and its use.  The last n-subtile's partials stay
        // in the ring for the next flush.
        auto compute = [&]() {
            if constexpr (P2) {
                static_for<0, 4 * NI>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    constexpr int ni = j / 4, mi = j % 4;
                    constexpr bool second = is_swiglu(EPI) && ni >= NI / 2;
                    if constexpr (WF4)
                        acc[mi][ni] = mfma16x16x128_fp4_e8m0(bfr[ni], af[mi], acc[mi][ni], eb4[ni], ea[mi]);
                    else
                        acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], af[mi], acc[mi][ni], second ? eb1 : eb0, ea[mi]);
                });
                return;
            }
            static_for<0, 4 * NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int ni = j / 4, mi = j % 4;
                if constexpr (j >= 4) {
                    constexpr int pn = ni - 1;
                    constexpr bool second = is_swiglu(EPI) && pn >= NI / 2;
                    acc[mi][pn] += ring[mi] * (second ? sc1[mi] : sc0[mi]);
                }
                ring[mi] = mfma16x16x128(bfr[ni], af[mi]);
                // keep this order: the scheduler would otherwise issue every
                // MFMA first, holding all partials live at once
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        using S0 = std::integral_constant<int, 0>;
        // Ping-pong over the two wave groups (waves 0-3 and 4-7, one of each
        // per SIMD): in every phase one group issues MFMAs while the other
        // reads its fragments from LDS.  A K block takes two phases; both
        // groups pass the same barriers in the same order.
        //   phase A (block kb): every wave has waited for its DMA of stage kb;
        //     DMA of kb + NS - 1 goes out (into the stage both groups finished
        //     with, the one of kb - 1); group 0 loads kb, group 1 multiplies kb - 1
        //   phase B: group 0 multiplies kb, group 1 loads kb
        // Stages 0 .. NS - 2 of the tile were issued before the previous epilogue.
        auto step0 = [&](auto st_c, int kb) {  // group 0: load kb, then multiply it
            constexpr int st = decltype(st_c)::value;
            wait_stage(kb);
            phase_barrier();
            if (kb + NS - 1 < nkb) issue(std::integral_constant<int, (st + NS - 1) % NS>{}, kb + NS - 1, cur);
            load(st_c, kb);
            phase_barrier();
            compute();
        };
        auto step1 = [&](auto st_c, int kb) {  // group 1: multiply kb - 1, then load kb
            constexpr int st = decltype(st_c)::value;
            wait_stage(kb);
            phase_barrier();
            if (kb + NS - 1 < nkb) issue(std::integral_constant<int, (st + NS - 1) % NS>{}, kb + NS - 1, cur);
            compute();
            phase_barrier();
            load(st_c, kb);
        };
        // unrolled by NS so that every stage index is a compile-time constant
        if (wave < 4) {
            for (int kb0 = 0; kb0 < nkb; kb0 += NS) {
                static_for<0, NS>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if (kb0 + i < nkb) step0(std::integral_constant<int, i>{}, kb0 + i);
                });
            }
        } else {
            // block 0 peeled: nothing to multiply yet (and the fragments are
            // never read before this group's first load)
            wait_stage(0);
            phase_barrier();
            if (NS - 1 < nkb) issue(std::integral_constant<int, NS - 1>{}, NS - 1, cur);
            phase_barrier();
            load(S0{}, 0);
            for (int kb0 = 1; kb0 < nkb; kb0 += NS) {
                static_for<0, NS>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if (kb0 + i < nkb) step1(std::integral_constant<int, (1 + i) % NS>{}, kb0 + i);
                });
            }
            compute();
        }
        flush();
        // every wave is done reading the stages and this tile's B scales: the
        // next tile's first NS - 1 stages and its B scales go out now, so
        // their latency overlaps this tile's epilogue (which writes from
        // registers and touches no stage)
        lds_barrier();
        const Tile ep = cur;
        if (t + G < total) {
            cur = tile_at(t + G);
            stage_bscale(cur);
            prologue(cur);
        }

        // ---------------------------------------------------------- epilogues
        // lane's outputs: row wm*64 + mi*16 + l15 of the tile, columns
        // wn*WN + ni*16 + 4*lg + v (v = 0..3) within the tile; written straight
        // from registers (each row's 4 lanes cover 16 contiguous columns)
        const int lg = lane >> 4;
        if constexpr (EPI == MOE_EPI_STORE_F32) {
            float* out = static_cast<float*>(g.out);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int64_t r = ep.row0 + wm * 64 + mi * 16 + l15;
                if (r >= ep.real_end) continue;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    *reinterpret_cast<v4f*>(out + r * N + ep.n0 + wn * WN + ni * 16 + 4 * lg) = acc[mi][ni];
            }
        } else if constexpr (EPI == MOE_EPI_STORE_BF16) {
            uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int64_t r = ep.row0 + wm * 64 + mi * 16 + l15;
                if (r >= ep.real_end) continue;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const v4f a = acc[mi][ni];
                    *reinterpret_cast<v2u*>(out + r * N + ep.n0 + wn * WN + ni * 16 + 4 * lg) =
                        v2u{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w)};
                }
            }
        } else if constexpr (is_swiglu(EPI)) {
            // n-subtiles 0, 1 are G and 2, 3 the U of the same h columns:
            // h column wn*32 + ni*16 + 4*lg + v of this tile's 128
            const int hcol0 = ep.nt * 128;
            v4f h[4][2];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int v = 0; v < 4; ++v) h[mi][ni][v] = silu(acc[mi][ni][v]) * acc[mi][ni + 2][v];
            if constexpr (EPI == MOE_EPI_SWIGLU_F32) {
                float* out = static_cast<float*>(g.out);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const int64_t r = ep.row0 + wm * 64 + mi * 16 + l15;
                    if (r >= ep.real_end) continue;
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        *reinterpret_cast<v4f*>(out + r * f + hcol0 + wn * 32 + ni * 16 + 4 * lg) = h[mi][ni];
                }
            } else {
                // row amax over this wave's 32 h columns (8 in-lane, then the 4
                // lane groups of the row), then across the 4 N waves via LDS
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    float m = 0.f;
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                        for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(h[mi][ni][v]));
                    m = fmaxf(m, __shfl_xor(m, 16));
                    m = fmaxf(m, __shfl_xor(m, 32));
                    if (lg == 0) rowmax[wn][wm * 64 + mi * 16 + l15] = m;
                }
                lds_barrier();
                uint8_t* out = static_cast<uint8_t*>(g.out);
                uint16_t* out2 = static_cast<uint16_t*>(g.out2);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const int rt = wm * 64 + mi * 16 + l15;
                    const int64_t r = ep.row0 + rt;
                    const float am = fmaxf(fmaxf(rowmax[0][rt], rowmax[1][rt]), fmaxf(rowmax[2][rt], rowmax[3][rt]));
                    if (r >= ep.real_end) continue;
                    const TileScale ts = tile_scale_t<P2>(am);
                    if (lg == 0 && wn == 0) g.out_s[(int64_t)ep.nt * g.row_cap + r] = ts.s;
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const int hc = hcol0 + wn * 32 + ni * 16 + 4 * lg;
                        const v4f hv = h[mi][ni];
                        *reinterpret_cast<uint32_t*>(out + r * f + hc) =
                            cvt_e4m3x4(hv.x * ts.inv, hv.y * ts.inv, hv.z * ts.inv, hv.w * ts.inv);
                        if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                            // G and U as bf16 for the backward
                            const v4f gv = acc[mi][ni], uv = acc[mi][ni + 2];
                            *reinterpret_cast<v2u*>(out2 + r * N + hc) = v2u{pack_bf16x2(gv.x, gv.y), pack_bf16x2(gv.z, gv.w)};
                            *reinterpret_cast<v2u*>(out2 + r * N + f + hc) = v2u{pack_bf16x2(uv.x, uv.y), pack_bf16x2(uv.z, uv.w)};
                        }
                    }
                }
            }
        }
        // the next tile's B scales (and this tile's row maxima) are settled
        // before any wave reads them
        lds_barrier();
    }
}

// ------------------------------------------------------------------ 256 x 256
// The same product on 256 x 256 block tiles.  A K step then moves 64 KB of
// operands for 16.8 MFLOP instead of 48 KB for 8.4 MFLOP (1.5x fewer bytes
// per MFMA from L2 and 25% fewer LDS fragment bytes).  Measured, the gain is
// smaller than that (hot-spot GEMM1 10%, ep8 GEMM1 2%): with every operand
// an L2 hit the kernel is only ~15% faster, while leaving out the global ->
// LDS DMA altogether makes it ~35% faster, so the DMA path, not bandwidth,
// bounds it.  The block tile is 288 x 256: an expert's rows take
// ceil(rows / 288) m-tiles, so the 400-576 rows of a training-shape expert
// stream its weights twice where 256-row tiles need three passes (the third
// for a tail of a few rows), and the 228-293 rows of an ep8 expert mostly fit
// one.  Eight waves (two per SIMD) as 2 (M) x 4 (N),
// each 144 x 64: its 144 accumulators leave no room for the ping-pong's
// all-fragments-at-once phase, so a wave holds its four B fragments of the K
// step and streams the nine A fragments, one 16-row subtile at a time, each
// followed by its four MFMAs (and, with fp32 scales, their rescale).  The two
// waves of a SIMD interleave on their own.  Two LDS stages (64 KB each) and
// one barrier per K step, placed before the step's last subtile: it frees the
// stage just read and publishes the next one, whose DMA was issued a step
// earlier, so a single vmcnt(0) per step suffices and loads may be skipped
// freely (A rows beyond the expert's padded segment are never fetched, and a
// wave whose rows are all padding issues no MFMAs).  Waves 0-3 issue all of
// a step's DMA (below), so waves 4-7 never stall on it.
// The tile height is a template parameter (MIT 16-row subtiles per wave: 9
// for 288 rows, 8 for 256); wide_mi() below picks it per variant.
constexpr int WBN = 256;

template <bool WF4, int WBM>
struct WideSmem {
    static constexpr int A_BYTES = WBM * GBK;
    static constexpr int B_BYTES = WBN * (WF4 ? GBK / 2 : GBK);
    static constexpr int S_BYTES = WBM * 4;
    static constexpr int BS_BYTES = WF4 ? WBN * 4 : 0;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES + BS_BYTES;
    static constexpr int TOTAL = 2 * STAGE;
};

// B operand read from a 64-bit transposing LDS load (gfx950
// ds_read_b64_tr_b8).  Within each 16-lane group the 16 addresses name 8-byte
// pieces P[s] (s = lane % 16) and lane i receives byte (i % 8) of
// P[2j + i / 8] as its byte j (measured): with P[2j + h] = bytes 8h .. 8h + 7 of
// K-row k0 + j of a [K][N]-ordered tile, lane i holds column i at K values
// k0 .. k0 + 7, in order, which is the MFMA operand's layout.
template <int OFF>
__device__ __forceinline__ v2u lds_tr8(uint32_t addr) {
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i_t* lds_v2i_ptr;
    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_ptr)(uintptr_t)(addr + OFF));
    return v2u{(uint32_t)r.x, (uint32_t)r.y};
}

// BKN: the weights come as [L, K, N] with scales [L, K/128, N/128] (the forward
// weights [out, in] of a dgrad product, which contracts over `out`), read
// without a transposed copy.  A K step's B tile is 128 K-rows of 256 bytes in
// LDS, row k's 16-byte chunk c stored at chunk c ^ f(k), f(k) = (k & 7) |
// ((k >> 4) & 1) << 3: the 32 rows one transposing load touches then spread
// over all 64 banks twice, the minimum for 512 bytes.
template <int EPI, bool P2, bool WF4, bool BKN, int MIT>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_wide_kernel(GemmArgs g) {
    constexpr int MI = MIT, NI = 4;  // 16 x 16 subtiles of a wave's (16 MI) x 64
    constexpr int WWR = 16 * MI;     // rows of a wave tile
    constexpr int WBM = 2 * WWR;     // rows of a block tile
    constexpr int WASEG = WBM / 32;  // 1 KB A segments (8 rows) per DMA wave and K step
    static_assert(MI == 8 || MI == 9, "256- or 288-row tiles");
    using SM = WideSmem<WF4, WBM>;
    static_assert(!WF4 || P2, "MXFP4 weights take the hardware-scale path");
    static_assert(!BKN || (!WF4 && !is_swiglu(EPI)), "[K, N] weights: FP8 dgrad products only");
    static_assert(!is_swiglu(EPI) || WBM == THIN_WBM, "thin-tile rule of the SwiGLU products");

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    __shared__ int tile_base[GMAXL + 1];
    __shared__ int64_t scan_tmp[GTHREADS];  // per-thread m-tiles (low word), thin tiles (high word)
    __shared__ float rowmax[4][WBM];
    __shared__ __attribute__((aligned(8))) float bscale[GMAXKB][2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int L = g.L, N = g.N, K = g.K;
    const int nkb = K / GBK;
    const int NT = N / WBN;
    const int f = N / 2;

    // ---- tile list: per expert ceil(real rows / 288) m-tiles x NT n-tiles.
    // g.thin: when the experts' thin last m-tiles (thin_rows_of) would add a
    // round of tiles for the G workgroups, they are left out here and the
    // K-split launches (gemm_thin.hip, the same rule) take them.
    {
        int loc[2], tloc[2];
        int64_t sum = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid * 2 + i;
            int m = 0, t = 0;
            if (e < L) {
                int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
                if (lo > g.row_cap) lo = g.row_cap;
                if (hi > g.row_cap) hi = g.row_cap;
                int64_t rows = g.counts[e];
                if (rows > hi - lo) rows = hi - lo;
                m = rows > 0 ? (int)((rows + WBM - 1) / WBM) : 0;
                t = (is_swiglu(EPI) && g.thin && thin_rows_of(rows) > 0) ? 1 : 0;
            }
            loc[i] = m;
            tloc[i] = t;
            sum += m + ((int64_t)t << 32);
        }
        scan_tmp[tid] = sum;
        __syncthreads();
        for (int off = 1; off < GTHREADS; off <<= 1) {
            const int64_t add = tid >= off ? scan_tmp[tid - off] : 0;
            __syncthreads();
            scan_tmp[tid] += add;
            __syncthreads();
        }
        const int64_t tot = scan_tmp[GTHREADS - 1];
        const bool split = thin_split_active((int)(tot & 0xFFFFFFFF), (int)(tot >> 32), NT, (int)gridDim.x);
        const int64_t before = scan_tmp[tid] - sum;
        int run = (int)(before & 0xFFFFFFFF) - (split ? (int)(before >> 32) : 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid * 2 + i;
            if (e < L) tile_base[e] = run * NT;
            run += loc[i] - (split ? tloc[i] : 0);
        }
        if (tid == 0) tile_base[L] = ((int)(tot & 0xFFFFFFFF) - (split ? (int)(tot >> 32) : 0)) * NT;
        __syncthreads();
    }
    const int total = tile_base[L];
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // fragment read offsets (stage-relative), as in the 128-row kernel with
    // 144-row wave tiles: A row wm*144 + mi*16 + l15, B row wn*64 + ni*16 + l15
    const int l15 = lane & 15, l7 = lane & 7, c0 = lane >> 4;
    const uint32_t a_rd0 = (wm * WWR + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t a_rd1 = (wm * WWR + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const int sw4 = ((l15 >> 1) ^ (l15 >> 3)) & 3;
    uint32_t b_rd0, b_rd1;
    if constexpr (BKN) {
        // K-row 16*c0 + l15/2 (+ 8, 64, 72 for the other three loads),
        // bytes 8*(l15 & 1) of the fragment's 16-column chunk; b_rd1 holds
        // 16 * ((4*wn) ^ f) and fragment ni's chunk term is b_rd1 ^ 16*ni
        const int fk = (l15 >> 1) | ((c0 & 1) << 3);
        b_rd0 = SM::A_BYTES + (16 * c0 + (l15 >> 1)) * 256 + 8 * (l15 & 1);
        b_rd1 = (uint32_t)(16 * ((4 * wn) ^ fk));
    } else {
        b_rd0 = WF4 ? SM::A_BYTES + (wn * 64 + l15) * 64 + ((c0 ^ sw4) << 4)
                    : SM::A_BYTES + (wn * 64 + l15) * 128 + ((c0 ^ l7) << 4);
        b_rd1 = SM::A_BYTES + (wn * 64 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    }
    const uint32_t bq_rd = SM::A_BYTES + SM::B_BYTES + SM::S_BYTES + (wn * 64 + l15) * 4 + c0;
    // A scales of a stage in row order (1152 bytes per K step): a lane's nine
    // rows wm*144 + mi*16 + l15 are 64 bytes apart
    const uint32_t s_rd = SM::A_BYTES + SM::B_BYTES + (wm * WWR + l15) * 4;

    struct Tile {
        int64_t row0, real_end, a_lim;  // first row, end of real rows, end of fetchable rows
        int nt, n0;
        const uint8_t* a_base;          // this wave's first A row, K block 0
        const uint8_t* b_base;
        const uint8_t* bsm;
        const float* s_base;
        const float* bs_lo;
        const float* bs_hi;
        int rot;
        int bnt;                        // 1: the expert has one m-tile, so no other tile reads these weight rows
        int na;                         // A DMA segments of this (DMA) wave inside a_lim (0..WASEG)
        int nmi;                        // 16-row subtiles of this wave with real rows (0..MI)
    };
    auto tile_at = [&](int t) {
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
        const int grp = local / (GROUP_M * NT);
        const int gm = min(GROUP_M, mt_e - grp * GROUP_M);
        const int in = local - grp * GROUP_M * NT;
        const int nt = in / gm, mt = grp * GROUP_M + (in - (in / gm) * gm);
        Tile ti;
        ti.row0 = (int64_t)g.offsets[e] + (int64_t)mt * WBM;
        ti.real_end = (int64_t)g.offsets[e] + g.counts[e];
        int64_t lim = g.offsets[e + 1];
        if (lim > g.row_cap) lim = g.row_cap;
        ti.a_lim = lim;
        if (ti.real_end > lim) ti.real_end = lim;
        {
            // DMA wave w (0-3) moves A rows [72w, 72w + 72) of the tile: the
            // segments of them inside the limit (a multiple of 8 rows away)
            const int64_t left = lim - (ti.row0 + (wave & 3) * 8 * WASEG);
            ti.na = left <= 0 ? 0 : (left >= 8 * WASEG ? WASEG : (int)(left / 8));
            const int64_t real = ti.real_end - (ti.row0 + wm * WWR);
            ti.nmi = real <= 0 ? 0 : (real >= WWR ? MI : (int)((real + 15) / 16));
        }
        ti.nt = nt;
        ti.n0 = nt * WBN;
        ti.a_base = g.a + (ti.row0 + (wave & 3) * 8 * WASEG) * K;
        int brow_w;
        if constexpr (is_swiglu(EPI)) {
            brow_w = ((wave & 1) ? f : 0) + nt * 128 + (wave >> 1) * 32;
        } else {
            brow_w = ti.n0 + wave * 32;
        }
        if constexpr (BKN)
            ti.b_base = g.b + (int64_t)e * K * N + ti.n0;  // K-row 0, the tile's first column
        else
            ti.b_base = WF4 ? g.b + ((int64_t)e * nkb * N + brow_w) * 64 : g.b + ((int64_t)e * N + brow_w) * K;
        ti.bsm = reinterpret_cast<const uint8_t*>(g.b_s) + ((int64_t)e * nkb * N + brow_w) * 4;
        ti.s_base = g.a_s + ti.row0;
        const float* bsx = g.b_s + (int64_t)e * (N / 128) * nkb;
        int blk0, blk1;
        if constexpr (is_swiglu(EPI)) {
            blk0 = nt;
            blk1 = f / 128 + nt;
        } else {
            blk0 = ti.n0 / 128;
            blk1 = blk0 + 1;
        }
        // [N/128, K/128] scales: a block's K run is contiguous; [K/128, N/128]
        // (BKN): it has stride N/128 (stage_bscale)
        ti.bs_lo = bsx + (BKN ? (int64_t)blk0 : (int64_t)blk0 * nkb);
        ti.bs_hi = bsx + (BKN ? (int64_t)blk1 : (int64_t)blk1 * nkb);
        ti.rot = ((mt & 1) * 2 + (nt & 3) * 2) % nkb;
        ti.bnt = mt_e == 1;
        return ti;
    };
    // the tile's two B scale rows (nkb <= GMAXKB <= 2 * GTHREADS: one load
    // per thread, from a uniform base, so no per-lane 64-bit pointer is formed)
    static_assert(GMAXKB <= 2 * GTHREADS, "one B scale per thread");
    auto stage_bscale = [&](const Tile& ti) {
        if constexpr (WF4) return;
        // waves 0-3: the low row, 4-7: the high one; the index comes from the
        // wave (uniform) and the lane id (recomputed), not a live register
        const int half = wave >> 2;
        const float* src = half ? ti.bs_hi : ti.bs_lo;
        const int kb = (wave & 3) * 64 + (int)__lane_id();
        if (kb < nkb) bscale[kb][half] = src[BKN ? kb * (N / 128) : kb];
    };
    const uint32_t bs_rd = lds_addr(&bscale[0][0]);
    const bool second_blk = !is_swiglu(EPI) && wn >= 2;

    // DMA lane offsets (1 KB segments of 8 fp8 rows / 16 fp4 rows, XOR
    // swizzled chunks as in the 128-row kernel)
    const int lr = lane >> 3;
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ lr) << 4);
    const uint32_t a_off0 = (uint32_t)(lr * K) + chunk;  // segment i adds 8*i*K
    uint32_t b_off0;
    if constexpr (WF4) {
        const int r4 = lane >> 2;
        b_off0 = (uint32_t)(r4 * 64) + (uint32_t)(((lane & 3) ^ (((r4 >> 1) ^ (r4 >> 3)) & 3)) << 4);  // segment i adds 1024*i
    } else {
        b_off0 = a_off0;
    }
    const uint32_t bs_off = (uint32_t)(lane * 4);
    // A scales: the tile's 288 row scales of a K block are 1152 contiguous
    // bytes (K-block-major layout): wave 0 moves rows 4l .. 4l + 3 with one
    // 16-byte-per-lane DMA, lanes 0-7 of wave 1 the last 32 rows (a 128-row
    // boundary never splits a lane's four)
    const uint32_t s_off = (uint32_t)(lane * 16);

    // issue_b / issue_a: the B (weights, with their fp4 scales) and A
    // (activations, with their scales) operands of a K block into a stage.
    // Waves 0-3, one per SIMD, issue all of a step's DMA: each its own B
    // share and that of wave + 4 (B rows 128 further, or 64 for the
    // interleaved SwiGLU blocks) and a quarter of the A rows, so that waves
    // 4-7 never stall on a DMA issue and keep the matrix cores busy meanwhile
    // (measured 2-7% faster than all eight waves issuing their own share).
    constexpr int BROW_P = is_swiglu(EPI) ? 64 : 128;
    const bool dma_self = wave < 4;
    const bool dma_pair = wave < 4;
    auto issue_b = [&](uint32_t sA, int kr, const Tile& ti) {
        const uint32_t sB = sA + SM::A_BYTES;
        auto one = [&](int w, int64_t brow_off) {
            if constexpr (WF4) {
                const uint8_t* bb = ti.b_base + (int64_t)kr * N * 64 + brow_off * 64;
                if (ti.bnt) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) dma16s_nt(bb, b_off0 + 1024 * i, sB + (w * 2 + i) * 1024);
                } else {
#pragma unroll
                    for (int i = 0; i < 2; ++i) dma16s(bb, b_off0 + 1024 * i, sB + (w * 2 + i) * 1024);
                }
                if (lane < 32)
                    dma4s(ti.bsm + (int64_t)kr * N * 4 + brow_off * 4, bs_off, sB + SM::B_BYTES + SM::S_BYTES + w * 128);
            } else if constexpr (BKN) {
                // K-rows 16w .. 16w + 15 of the step, 4 per 1 KB segment:
                // lane l fills chunk position l % 16 of row 16w + 4i + l/16
                // with the global chunk (l % 16) ^ f(row)
                const uint8_t* bb = ti.b_base + ((int64_t)kr * GBK + 16 * w) * N;
                const uint32_t l = (uint32_t)__lane_id();
                const uint32_t rsub = l >> 4, pos = l & 15, fw = (uint32_t)((w & 1) << 3);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t fk = (uint32_t)(4 * (i & 1)) + rsub + fw;
                    dma16s(bb, (uint32_t)((4 * i) * N) + rsub * (uint32_t)N + ((pos ^ fk) << 4),
                           sB + (w * 4 + i) * 1024);
                }
            } else {
                const uint8_t* bb = ti.b_base + kr * GBK + brow_off * K;
                // weight rows that only this tile reads (one m-tile in the
                // expert) stream past the caches: measured 2-3% faster at that
                // shape, and 4-5% slower where a second m-tile re-reads them
                if (ti.bnt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) dma16s_nt(bb, b_off0 + (uint32_t)(8 * i * K), sB + (w * 4 + i) * 1024);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) dma16s(bb, b_off0 + (uint32_t)(8 * i * K), sB + (w * 4 + i) * 1024);
                }
            }
        };
        if (dma_self) one(wave, 0);
        if (dma_pair) one(wave + 4, BROW_P);
    };
    auto issue_a = [&](uint32_t sA, int kr, const Tile& ti) {
        if (dma_self) {
            // segments in groups of four: the group's row offset goes on the
            // wave-uniform base, so only four per-lane offsets are formed
            const uint8_t* ab = ti.a_base + kr * GBK;
            static_for<0, WASEG>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if (i < ti.na)
                    dma16s(ab + (int64_t)(32 * (i / 4)) * K, a_off0 + (uint32_t)(8 * (i % 4) * K),
                           sA + (wave * WASEG + i) * 1024);
            });
        }
        if (wave == 0 && ti.row0 + 4 * lane < ti.a_lim)
            dma16s(ti.s_base + (int64_t)kr * g.row_cap, s_off, sA + SM::A_BYTES + SM::B_BYTES);
        if (wave == 1 && lane < (WBM - 256) / 4 && ti.row0 + 256 + 4 * lane < ti.a_lim)
            dma16s(ti.s_base + (int64_t)kr * g.row_cap + 256, s_off, sA + SM::A_BYTES + SM::B_BYTES + 1024);
    };
    auto krot = [&](int kb, const Tile& ti) {
        int kr = kb + ti.rot;
        if (kr >= nkb) kr -= nkb;
        return kr;
    };
    auto lds_barrier = [&]() {
        wait_lgkm0();
        phase_barrier();
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    int t = lb;
    Tile cur;
    if (t < total) {
        cur = tile_at(t);
        stage_bscale(cur);
        issue_b(sbase, krot(0, cur), cur);
        issue_a(sbase, krot(0, cur), cur);
    }
    for (; t < total; t += G) {
        v4f acc[MI][NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;
        const int nmi = cur.nmi;

        // Operands of the current K step held in registers: B fragments (and
        // fp4 scale codes), A and B scales, and the first A fragment.
        v8i bfr[NI];
        int eb4[NI];
        uint32_t sac = 0;  // A scale of the current subtile's rows (this lane's)
        uint32_t sbx = 0, sby = 0;
        v8i afc;
        auto read_b = [&](auto nc, uint32_t pb0, uint32_t pb1, uint32_t pbs) {
            constexpr int ni = decltype(nc)::value;
            if constexpr (WF4) {
                const u32x4 z4 = {0u, 0u, 0u, 0u};
                bfr[ni] = join8(lds16<ni * 1024>(pb0), z4);
                eb4[ni] = (int)lds1<ni * 64>(pbs);
            } else if constexpr (BKN) {
                // K values 16c0 .. +7, +8 .. +15, 16c0 + 64 .. +71, +72 .. +79
                const uint32_t pa = pb0 + (b_rd1 ^ (uint32_t)(16 * ni));
                const v2u r0 = lds_tr8<0>(pa), r1 = lds_tr8<2048>(pa);
                const v2u r2 = lds_tr8<16384>(pa), r3 = lds_tr8<18432>(pa);
                bfr[ni] = v8i{(int)r0.x, (int)r0.y, (int)r1.x, (int)r1.y, (int)r2.x, (int)r2.y, (int)r3.x, (int)r3.y};
            } else {
                bfr[ni] = join8(lds16<ni * 2048>(pb0), lds16<ni * 2048>(pb1));
            }
        };
        // the step's B block scales and subtile 0's A scale; the A scale of
        // subtile mi + 1 is read with its fragment while mi multiplies
        auto read_scales = [&](uint32_t ps, uint32_t bsa) {
            const v2u sbv = lds8<0>(bsa);
            sbx = sbv.x;
            sby = sbv.y;
            sac = lds4<0>(ps);
        };
        auto read_a = [&](auto mc, uint32_t pa0, uint32_t pa1) {
            constexpr int mi = decltype(mc)::value;
            return join8(lds16<mi * 2048>(pa0), lds16<mi * 2048>(pa1));
        };
        // every operand of a step, from the stage at LDS address sX
        auto read_step = [&](uint32_t sX, int kr) {
            uint32_t pb0 = sX + b_rd0, pb1 = sX + b_rd1, pbs = sX + bq_rd, ps = sX + s_rd;
            uint32_t pa0 = sX + a_rd0, pa1 = sX + a_rd1, bsa = bs_rd + kr * 8;
            pin(pb0); pin(pb1); pin(pbs); pin(ps); pin(pa0); pin(pa1); pin(bsa);
            static_for<0, NI>([&](auto nc) { read_b(nc, pb0, pb1, pbs); });
            read_scales(ps, bsa);
            afc = read_a(std::integral_constant<int, 0>{}, pa0, pa1);
        };
        // four MFMAs of 16-row subtile mi on fragment af; with fp32 scales
        // their fresh partials are rescaled into the accumulators
        auto subtile = [&](auto mc, const v8i& af, uint32_t sa_bits) {
            constexpr int mi = decltype(mc)::value;
            if constexpr (P2) {
                const int ea = (int)(sa_bits >> 23);
                const int eb0 = (int)((second_blk ? sby : sbx) >> 23), eb1 = (int)(sby >> 23);
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    constexpr bool second = is_swiglu(EPI) && ni >= NI / 2;
                    if constexpr (WF4)
                        acc[mi][ni] = mfma16x16x128_fp4_e8m0(bfr[ni], af, acc[mi][ni], eb4[ni], ea);
                    else
                        acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], af, acc[mi][ni], second ? eb1 : eb0, ea);
                });
            } else {
                const float sa = __uint_as_float(sa_bits);
                const float s0 = sa * __uint_as_float(second_blk ? sby : sbx);
                const float s1 = sa * __uint_as_float(sby);
                v4f p[NI];
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    p[ni] = mfma16x16x128(bfr[ni], af);
                });
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    constexpr bool second = is_swiglu(EPI) && ni >= NI / 2;
                    acc[mi][ni] += p[ni] * (second ? s1 : s0);
                });
            }
        };

        // One K step from stage st.  Subtiles 0-6 run straight-line code (the
        // compiler counts the outstanding LDS reads exactly; scheduling
        // barriers keep the order, since hoisted, the eight A fragments would
        // not fit next to the accumulators), each reading the next subtile's
        // A fragment while it multiplies.  Then every LDS read of stage st is
        // done, and once this wave's DMA of step kb + 1 has landed one
        // barrier both frees stage st and publishes stage st ^ 1: the DMA of
        // step kb + 2 goes out, and the last subtile's MFMAs run while the
        // next step's B fragments, scales and first A fragment are read (each
        // B fragment right after the MFMA that last uses the old one).  A
        // wave whose 128 rows are all padding skips the MFMAs and reads; a
        // partly filled one runs all subtiles (a second, guarded copy of this
        // code costs the register allocation hundreds of spills).
        auto kstep = [&](auto st_c, int kb) {
            constexpr int st = decltype(st_c)::value;
            const uint32_t sA = sbase + (uint32_t)(st * SM::STAGE);
            const uint32_t sN = sbase + (uint32_t)((st ^ 1) * SM::STAGE);
            if (nmi > 0) {
                uint32_t pa0 = sA + a_rd0, pa1 = sA + a_rd1, ps = sA + s_rd;
                pin(pa0); pin(pa1); pin(ps);
                static_for<0, MI - 1>([&](auto mc) {
                    constexpr int mi = decltype(mc)::value;
                    const v8i afn = read_a(std::integral_constant<int, mi + 1>{}, pa0, pa1);
                    const uint32_t san = lds4<(mi + 1) * 64>(ps);
                    subtile(mc, afc, sac);
                    __builtin_amdgcn_sched_barrier(0);
                    afc = afn;
                    sac = san;
                });
            }
            wait_vmcnt<0>();
            lds_barrier();
            if (kb + 2 < nkb) {
                const int kr2 = krot(kb + 2, cur);
                issue_b(sA, kr2, cur);
                issue_a(sA, kr2, cur);
            }
            if (nmi > 0) {
                // reads of the step after the tile's last one fetch unused
                // values (krot keeps the B-scale index in range)
                uint32_t pb0 = sN + b_rd0, pb1 = sN + b_rd1, pbs = sN + bq_rd;
                pin(pb0); pin(pb1); pin(pbs);
                constexpr int mi = MI - 1;
                if constexpr (P2) {
                    const int ea = (int)(sac >> 23);
                    const int eb0 = (int)((second_blk ? sby : sbx) >> 23), eb1 = (int)(sby >> 23);
                    static_for<0, NI>([&](auto nc) {
                        constexpr int ni = decltype(nc)::value;
                        constexpr bool second = is_swiglu(EPI) && ni >= NI / 2;
                        if constexpr (WF4)
                            acc[mi][ni] = mfma16x16x128_fp4_e8m0(bfr[ni], afc, acc[mi][ni], eb4[ni], ea);
                        else
                            acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], afc, acc[mi][ni], second ? eb1 : eb0, ea);
                        read_b(nc, pb0, pb1, pbs);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                } else {
                    const float sa = __uint_as_float(sac);
                    const float s0 = sa * __uint_as_float(second_blk ? sby : sbx);
                    const float s1 = sa * __uint_as_float(sby);
                    v4f p[NI];
                    static_for<0, NI>([&](auto nc) {
                        constexpr int ni = decltype(nc)::value;
                        p[ni] = mfma16x16x128(bfr[ni], afc);
                        read_b(nc, pb0, pb1, pbs);
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    static_for<0, NI>([&](auto nc) {
                        constexpr int ni = decltype(nc)::value;
                        constexpr bool second = is_swiglu(EPI) && ni >= NI / 2;
                        acc[mi][ni] += p[ni] * (second ? s1 : s0);
                    });
                }
                uint32_t ps = sN + s_rd, pa0 = sN + a_rd0, pa1 = sN + a_rd1, bsa = bs_rd + krot(kb + 1, cur) * 8;
                pin(ps); pin(pa0); pin(pa1); pin(bsa);
                read_scales(ps, bsa);
                afc = read_a(std::integral_constant<int, 0>{}, pa0, pa1);
            }
        };

        // stage 0 (step 0) has landed: step 1 goes out, step 0's operands are read
        wait_vmcnt<0>();
        lds_barrier();
        if (nkb > 1) {
            const int kr1 = krot(1, cur);
            issue_b(sbase + SM::STAGE, kr1, cur);
            issue_a(sbase + SM::STAGE, kr1, cur);
        }
        if (nmi > 0) read_step(sbase, krot(0, cur));
        for (int kb0 = 0; kb0 < nkb; kb0 += 2) {
            kstep(std::integral_constant<int, 0>{}, kb0);
            if (kb0 + 1 < nkb) kstep(std::integral_constant<int, 1>{}, kb0 + 1);
        }
        // all stages and this tile's B scales are free: the next tile's first
        // step goes out now and overlaps the epilogue
        const Tile ep = cur;
        if (t + G < total) {
            cur = tile_at(t + G);
            stage_bscale(cur);
            issue_b(sbase, krot(0, cur), cur);
            issue_a(sbase, krot(0, cur), cur);
        }

        // the epilogue's lane indices, from an opaque copy of the lane id: its
        // per-lane row and address terms are then formed here, once per tile,
        // instead of being hoisted above the K loop, where they held registers
        // through it (the SwiGLU variants spilled them)
        const int lane_e = (int)opaque((uint32_t)lane);
        const int lg = lane_e >> 4, l15e = lane_e & 15;
        if constexpr (EPI == MOE_EPI_STORE_F32) {
            float* out = static_cast<float*>(g.out);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int64_t r = ep.row0 + wm * WWR + mi * 16 + l15e;
                if (r >= ep.real_end) continue;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    *reinterpret_cast<v4f*>(out + r * N + ep.n0 + wn * 64 + ni * 16 + 4 * lg) = acc[mi][ni];
            }
        } else if constexpr (EPI == MOE_EPI_STORE_BF16) {
            // two cross-lane swaps per pair of n-subtiles regroup a row's
            // columns so that lane group lg holds columns 8lg .. 8lg + 7 of
            // each 32-column pair: one 16-byte store where the MFMA layout
            // gives two 8-byte ones (half the store instructions, each of
            // which costs the texture addresser as much as a 1 KB load).  The
            // swaps run on every lane; only the stores skip padding rows.
            uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int64_t r = ep.row0 + wm * WWR + mi * 16 + l15e;
                uint32_t x[NI], y[NI];  // columns (0, 1) and (2, 3) of each subtile, packed bf16
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const v4f a = acc[mi][ni];
                    x[ni] = pack_bf16x2(a.x, a.y);
                    y[ni] = pack_bf16x2(a.z, a.w);
                }
#pragma unroll
                for (int ni = 0; ni < NI; ni += 2) {
                    swap32(x[ni], x[ni + 1]);
                    swap32(y[ni], y[ni + 1]);
                    swap16(x[ni], x[ni + 1]);
                    swap16(y[ni], y[ni + 1]);
                }
                if (r >= ep.real_end) continue;
#pragma unroll
                for (int h = 0; h < NI / 2; ++h)
                    *reinterpret_cast<u32x4*>(out + r * N + ep.n0 + wn * 64 + 32 * h + 8 * lg) =
                        u32x4{x[2 * h], y[2 * h], x[2 * h + 1], y[2 * h + 1]};
            }
        } else if constexpr (is_swiglu(EPI)) {
            const int hcol0 = ep.nt * 128;
            if constexpr (EPI == MOE_EPI_SWIGLU_F32) {
                float* out = static_cast<float*>(g.out);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int64_t r = ep.row0 + wm * WWR + mi * 16 + l15e;
                    if (r >= ep.real_end) continue;
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        v4f h;
#pragma unroll
                        for (int v = 0; v < 4; ++v) h[v] = silu(acc[mi][ni][v]) * acc[mi][ni + 2][v];
                        *reinterpret_cast<v4f*>(out + r * f + hcol0 + wn * 32 + ni * 16 + 4 * lg) = h;
                    }
                }
            } else {
                // h overwrites the U accumulators once G and U are saved; the
                // row amax goes across the 4 N waves through LDS
                uint16_t* out2 = static_cast<uint16_t*>(g.out2);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int64_t r = ep.row0 + wm * WWR + mi * 16 + l15e;
                    float m = 0.f;
                    if constexpr (EPI == MOE_EPI_SWIGLU_Q8_SAVE) {
                        // G and U as bf16, regrouped like the bf16 store
                        // epilogue: one 16-byte store each per lane and row
                        uint32_t gx[2], gy[2], ux[2], uy[2];
#pragma unroll
                        for (int ni = 0; ni < 2; ++ni) {
                            const v4f gv = acc[mi][ni], uv = acc[mi][ni + 2];
                            gx[ni] = pack_bf16x2(gv.x, gv.y);
                            gy[ni] = pack_bf16x2(gv.z, gv.w);
                            ux[ni] = pack_bf16x2(uv.x, uv.y);
                            uy[ni] = pack_bf16x2(uv.z, uv.w);
                        }
                        swap32(gx[0], gx[1]);
                        swap32(gy[0], gy[1]);
                        swap32(ux[0], ux[1]);
                        swap32(uy[0], uy[1]);
                        swap16(gx[0], gx[1]);
                        swap16(gy[0], gy[1]);
                        swap16(ux[0], ux[1]);
                        swap16(uy[0], uy[1]);
                        if (r < ep.real_end) {
                            const int hc = hcol0 + wn * 32 + 8 * lg;
                            *reinterpret_cast<u32x4*>(out2 + r * N + hc) = u32x4{gx[0], gy[0], gx[1], gy[1]};
                            *reinterpret_cast<u32x4*>(out2 + r * N + f + hc) = u32x4{ux[0], uy[0], ux[1], uy[1]};
                        }
                    }
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const v4f gv = acc[mi][ni], uv = acc[mi][ni + 2];
                        v4f h;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            h[v] = silu(gv[v]) * uv[v];
                            m = fmaxf(m, fabsf(h[v]));
                        }
                        acc[mi][ni + 2] = h;
                    }
                    m = fmaxf(m, __shfl_xor(m, 16));
                    m = fmaxf(m, __shfl_xor(m, 32));
                    if (lg == 0) rowmax[wn][wm * WWR + mi * 16 + l15e] = m;
                }
                lds_barrier();
                uint8_t* out = static_cast<uint8_t*>(g.out);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int rt = wm * WWR + mi * 16 + l15e;
                    const int64_t r = ep.row0 + rt;
                    const float am = fmaxf(fmaxf(rowmax[0][rt], rowmax[1][rt]), fmaxf(rowmax[2][rt], rowmax[3][rt]));
                    const TileScale ts = tile_scale_t<P2>(am);
                    // the 4-code groups regrouped like the bf16 epilogue's
                    // column pairs: 8 consecutive codes per lane, one store
                    uint32_t z[2];
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const v4f hv = acc[mi][ni + 2];
                        z[ni] = cvt_e4m3x4(hv.x * ts.inv, hv.y * ts.inv, hv.z * ts.inv, hv.w * ts.inv);
                    }
                    swap32(z[0], z[1]);
                    swap16(z[0], z[1]);
                    if (r >= ep.real_end) continue;
                    if (lg == 0 && wn == 0) g.out_s[(int64_t)ep.nt * g.row_cap + r] = ts.s;
                    *reinterpret_cast<v2u*>(out + r * f + hcol0 + wn * 32 + 8 * lg) = v2u{z[0], z[1]};
                }
            }
        }
        // row maxima read and the next tile's B scales written before reuse
        lds_barrier();
    }
}

// Every variant takes 288-row tiles and compiles without spilled registers
// (218-250 VGPRs).
template <int EPI, bool P2, bool WF4, bool BKN>
constexpr int wide_mi() {
    return 9;
}

template <int EPI, bool P2, bool WF4, bool BKN>
static void go_wide(const GemmArgs& a, int grid, hipStream_t stream) {
    gemm_wide_kernel<EPI, P2, WF4, BKN, wide_mi<EPI, P2, WF4, BKN>()><<<dim3(grid), dim3(GTHREADS), 0, stream>>>(a);
}

template <int EPI>
static int launch_wide(const GemmArgs& a, bool p2, bool wf4, hipStream_t stream, bool bkn = false) {
    const int ncu = num_cus();
    const int grid = (ncu + 7) / 8 * 8;
    if constexpr (EPI == MOE_EPI_STORE_BF16 || EPI == MOE_EPI_STORE_F32) {
        if (bkn) {
            p2 ? go_wide<EPI, true, false, true>(a, grid, stream) : go_wide<EPI, false, false, true>(a, grid, stream);
            MOE_LAUNCH_CHECK("gemm_wide_kernel");
            return MOE_OK;
        }
    }
    if (wf4)
        go_wide<EPI, true, true, false>(a, grid, stream);
    else if (p2)
        go_wide<EPI, true, false, false>(a, grid, stream);
    else
        go_wide<EPI, false, false, false>(a, grid, stream);
    MOE_LAUNCH_CHECK("gemm_wide_kernel");
    return MOE_OK;
}

template <int BN, int EPI>
static int launch_gemm(const GemmArgs& a, bool p2, bool wf4, bool wide, hipStream_t stream, bool bkn = false) {
    if constexpr (BN == 256) {
        if (wide) return launch_wide<EPI>(a, p2, wf4, stream, bkn);
    }
    const int ncu = num_cus();
    const int grid = (ncu + 7) / 8 * 8;  // one 512-thread block per CU (LDS bound), persistent
    if (wf4)
        gemm_fp8_kernel<BN, EPI, true, true><<<dim3(grid), dim3(GTHREADS), 0, stream>>>(a);
    else if (p2)
        gemm_fp8_kernel<BN, EPI, true, false><<<dim3(grid), dim3(GTHREADS), 0, stream>>>(a);
    else
        gemm_fp8_kernel<BN, EPI, false, false><<<dim3(grid), dim3(GTHREADS), 0, stream>>>(a);
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
    const bool p2 = (epilogue & MOE_SCALE_POW2) != 0;
    const bool wf4 = (epilogue & MOE_WEIGHT_MXFP4) != 0;
    const bool tile128 = (epilogue & MOE_GEMM_TILE128) != 0;
    const bool bkn = (epilogue & MOE_GEMM_B_KN) != 0;
    const bool thin = (epilogue & MOE_GEMM_THIN_SPLIT) != 0;
    epilogue &= ~(MOE_SCALE_POW2 | MOE_WEIGHT_MXFP4 | MOE_GEMM_TILE128 | MOE_GEMM_B_KN | MOE_GEMM_THIN_SPLIT);
    MOE_REQUIRE(!wf4 || p2, MOE_ERR_UNSUPPORTED, "grouped_gemm: MXFP4 weights need MOE_SCALE_POW2 activations");
    MOE_REQUIRE(!bkn || (!wf4 && !tile128 && N % 256 == 0 &&
                         (epilogue == MOE_EPI_STORE_BF16 || epilogue == MOE_EPI_STORE_F32)),
                MOE_ERR_UNSUPPORTED,
                "grouped_gemm: [K, N] weights need FP8 weights, 256 x 256 tiles (N %% 256 == 0) and a store epilogue");
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
    MOE_REQUIRE(!thin || (swiglu && !wf4 && !tile128), MOE_ERR_UNSUPPORTED,
                "grouped_gemm: MOE_GEMM_THIN_SPLIT needs a SwiGLU epilogue, FP8 weights and 288-row tiles");
    MOE_REQUIRE(!thin || out3, MOE_ERR_NULL, "grouped_gemm: MOE_GEMM_THIN_SPLIT needs the workspace in out3");
    if (row_cap == 0) return MOE_OK;
    GemmArgs ga{a, a_s, b, b_s, counts, offsets, L, row_cap, N, K, epi_in, out, out_s, out2, out2_s, out3, out3_s,
                thin ? 1 : 0};
    const bool wide = N % 256 == 0;
    switch (epilogue) {
        case MOE_EPI_STORE_BF16:
            return wide ? launch_gemm<256, MOE_EPI_STORE_BF16>(ga, p2, wf4, !tile128, stream, bkn)
                        : launch_gemm<128, MOE_EPI_STORE_BF16>(ga, p2, wf4, !tile128, stream);
        case MOE_EPI_STORE_F32:
            return wide ? launch_gemm<256, MOE_EPI_STORE_F32>(ga, p2, wf4, !tile128, stream, bkn)
                        : launch_gemm<128, MOE_EPI_STORE_F32>(ga, p2, wf4, !tile128, stream);
        case MOE_EPI_SWIGLU_Q8:
        case MOE_EPI_SWIGLU_Q8_SAVE:
        case MOE_EPI_SWIGLU_F32: {
            const int rc = epilogue == MOE_EPI_SWIGLU_Q8
                               ? launch_gemm<256, MOE_EPI_SWIGLU_Q8>(ga, p2, wf4, !tile128, stream)
                           : epilogue == MOE_EPI_SWIGLU_Q8_SAVE
                               ? launch_gemm<256, MOE_EPI_SWIGLU_Q8_SAVE>(ga, p2, wf4, !tile128, stream)
                               : launch_gemm<256, MOE_EPI_SWIGLU_F32>(ga, p2, wf4, !tile128, stream);
            if (rc != MOE_OK || !thin) return rc;
            return moe_thin_launch(a, a_s, b, b_s, counts, offsets, L, row_cap, N, K, epilogue, p2,
                                   static_cast<float*>(out3), out, out_s, out2, stream);
        }
    }
    return fail(MOE_ERR_UNSUPPORTED, "grouped_gemm: epilogue %d", epilogue);
}

extern "C" int moe_grouped_gemm_thin_workspace(int32_t L, int32_t N, int32_t K, size_t* bytes) {
    MOE_REQUIRE(bytes, MOE_ERR_NULL, "grouped_gemm_thin_workspace: NULL bytes");
    MOE_REQUIRE(L >= 1 && L <= GMAXL && N > 0 && N % 256 == 0 && K > 0 && K % 128 == 0 && K / 128 <= GMAXKB,
                MOE_ERR_SHAPE, "grouped_gemm_thin_workspace: bad L=%d, N=%d or K=%d", L, N, K);
    *bytes = moe_thin_workspace_bytes(L, N, K);
    return MOE_OK;
}
