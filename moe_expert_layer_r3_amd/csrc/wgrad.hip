// Weight-gradient grouped GEMM ("RL at 1T scale", section "FP8 Training":
// block-scaled FP8 trainer GEMMs; the backward re-quantises each operand along
// its contraction axis, here the token axis).
//
// For every local expert e and its padded row segment [offsets[e], offsets[e+1]):
//   dW[e][m, n] = sum over 128-row token blocks b of the segment of
//                 aT_s[b, m] * bT_s[b, n] * (aT[m, 128b:128b+128] . bT[n, 128b:128b+128])
// aT and bT are the operands transposed and tiled by token block: aT[b][m][i]
// is token 128b + i of row m ([row_cap/128, M, 128] bytes), so one K step of a
// 128-row tile is a single contiguous 16 KB piece (with a plain [M, row_cap]
// layout the 128 rows sit a power-of-two multiple apart and thrash the L2's
// sets).  Scales are one per (row, token block) for both operands, stored
// token-block-major, so one block's scales of a tile are contiguous too.
//
// Shape of the problem: an expert's segment is short (a few hundred tokens,
// a handful of K steps) while its output M x N is large, so a tile does little
// MFMA work per byte of bf16 it writes, and the operand stream is bounded by
// the requests a CU can keep in flight to L2 (bytes per step / latency), not
// by bandwidth.  The kernel is built around that:
//   * 128 x 256 tiles where N allows (48 KB of operands per K step for 16
//     MFMAs per wave; 128 x 128 needs 32 KB for 8);
//   * each workgroup runs ONE stream of K steps over all of its tiles; the
//     three-stage LDS DMA ring runs two steps ahead across tile boundaries, so
//     a new tile never starts on an empty pipeline;
//   * a finished tile is stored straight from registers while the next
//     tile's loads are in flight.  Two cross-lane swaps first regroup each
//     row's columns so that a lane holds 8 consecutive bf16, and a pair
//     exchange between the lanes of adjacent rows lets every store
//     instruction write whole 128-byte lines.  Stores and loads share the
//     wave's vector-memory counter, so every wait counts the stores issued
//     after the awaited stage and never drains them;
//   * tiles of experts without rows are not in the stream: their dW = 0 is
//     written by a plain fill after it.
// Three kernels share this: the streaming one (wgrad_fp8_kernel, both
// operands through the ring), one that keeps an m-tile's A operand in LDS
// for experts of up to ARES_KB token blocks (wgrad_ares_kernel: only B
// streams), and 256 x 256 tiles for power-of-two scales (wgrad_wide_kernel).
// Where the A-resident kernel applies, a second launch of the streaming one
// takes the experts with more token blocks.
// The K step itself is the forward grouped GEMM's: 8 waves in two ping-pong
// groups (one of each per SIMD), conflict-free swizzled fragments,
// weights-first MFMA operand order; both operands carry per-row scales, so the
// factor of a partial is sA[row] * sB[column], formed as the partial is added.
// With power-of-two scales (P2) that factor is exactly what the block-scaled
// MFMA applies per operand row: each lane passes the E8M0 exponents of its A
// row and its B row, and the MFMA accumulates in place (no rescale on the VALU).
#include "mfma_common.hpp"

namespace moe {

// dW leaves with streaming (non-temporal) stores: it is written once and not
// read again in the step, so its lines need not stay dirty in L2 and the
// last-level cache for the kernels that follow
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

constexpr int WBM = 128;  // tile rows (M); tile columns BN = 256 or 128
constexpr int WBK = 128;  // tokens per K step (one quantisation block)
constexpr int WTHREADS = 512;
constexpr int WMAXL = 1024;

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
    int nfast;  // 1: n-tiles vary fastest in the tile order (B is the smaller operand)
    int gf;     // fast-index tiles per group (divides that index's tile count)
    uint16_t* dW;
    int kb_min, kb_max;  // this launch takes the experts with kb_min..kb_max token blocks
    int zfill;           // 1: this launch also writes dW = 0 for experts without rows
};

// Experts whose segment holds kb_min .. kb_max token blocks, in order (wave
// 0): tab[0] = their count, tab_x[i] = e | nkb << 10, tab_lo[i] = first row.
__device__ __forceinline__ void build_expert_table(const WgradArgs& g, int64_t rcap, int wave, int lane, int* tab,
                                                   int* tab_x, int* tab_lo) {
    if (wave != 0) return;
    int cnt = 0;
    for (int c = 0; c < g.L; c += 64) {
        const int e = c + lane;
        int64_t lo = 0, hi = 0;
        if (e < g.L) {
            lo = g.offsets[e];
            hi = g.offsets[e + 1];
            lo = lo < 0 ? 0 : (lo > rcap ? rcap : lo);
            hi = hi > rcap ? rcap : hi;
        }
        const int nkb = hi > lo ? (int)((hi - lo) / WBK) : 0;
        const bool take = nkb > 0 && nkb >= g.kb_min && nkb <= g.kb_max;
        const uint64_t m = __ballot(take);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (take) {
            tab_x[cnt + below] = e | (nkb << 10);
            tab_lo[cnt + below] = (int)lo;
        }
        cnt += __popcll(m);
    }
    if (lane == 0) tab[0] = cnt;
}

// dW = 0 for the experts without a token block (when this launch owns the fill)
__device__ __forceinline__ void zero_fill_empty(const WgradArgs& g, int tid) {
    if (!g.zfill) return;
    const int64_t rcap = g.row_cap;
    const int64_t chunks = (int64_t)g.M * g.N / 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int e = 0; e < g.L; ++e) {
        int64_t lo = g.offsets[e], hi = g.offsets[e + 1];
        lo = lo < 0 ? 0 : (lo > rcap ? rcap : lo);
        hi = hi > rcap ? rcap : hi;
        if (hi - lo >= WBK) continue;
        uint16_t* d = g.dW + (int64_t)e * g.M * g.N;
        for (int64_t c = (int64_t)blockIdx.x * WTHREADS + tid; c < chunks; c += (int64_t)gridDim.x * WTHREADS)
            st_stream(reinterpret_cast<u32x4*>(d + c * 8), z);
    }
}

template <int BN>
struct WgradSmem {
    static constexpr int A_BYTES = WBM * WBK;
    static constexpr int B_BYTES = BN * WBK;
    static constexpr int SA_BYTES = WBM * 4;
    static constexpr int SB_BYTES = BN * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int TAB = 3 * STAGE;  // experts with rows: count, packed id|nkb, lo
    static constexpr int TOTAL = TAB + (1 + 2 * WMAXL) * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS");
};

// vmcnt wait for a count known only at run time; n is one of the few sums of
// NLD (a stage's loads) and NST (a tile's stores) the loop produces.
template <int NLD, int NST>
__device__ __forceinline__ void wait_younger(int n) {
    if (n == NLD) wait_vmcnt<NLD>();
    else if (n == NLD + NST) wait_vmcnt<NLD + NST>();
    else if (n == NLD + 2 * NST) wait_vmcnt<NLD + 2 * NST>();
    else if (n == NST) wait_vmcnt<NST>();
    else if (n == 2 * NST) wait_vmcnt<2 * NST>();
    else wait_vmcnt<0>();
}

template <int BN, bool P2>
__global__ __launch_bounds__(WTHREADS, 1) void wgrad_fp8_kernel(WgradArgs g) {
    using SM = WgradSmem<BN>;
    constexpr int WN = BN / 4;             // wave tile columns
    constexpr int NI = WN / 16;            // n-subtiles per wave
    constexpr int ASEG = WBM / 64;         // 1 KB A segments (8 rows) per wave per stage
    constexpr int BSEG = BN / 64;          // 1 KB B segments per wave per stage
    constexpr int SROWS = BN / 8;          // B scales loaded per wave
    constexpr int NLD = ASEG + BSEG + 2;   // DMA instructions per wave per stage (+ A and B scales)
    constexpr int NST = 2 * NI;            // 16-byte stores per wave per tile
    static_assert(SROWS <= 64 && 2 * NLD + 2 * NST < 64, "DMA lanes, vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    int* const tab = reinterpret_cast<int*>(smem + SM::TAB);
    int* const tab_x = tab + 1;           // e | nkb << 10
    int* const tab_lo = tab + 1 + WMAXL;  // first row of the segment

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t rcap = g.row_cap;
    const int M = g.M, N = g.N;
    const int MT = M / WBM, NT = N / BN, TPE = MT * NT;
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // experts of this launch (token block counts kb_min..kb_max), in order
    build_expert_table(g, rcap, wave, lane, tab, tab_x, tab_lo);
    __syncthreads();
    const int Lne = __builtin_amdgcn_readfirstlane(tab[0]);
    const int total = Lne * TPE;  // tiles with K work, expert-major, then n-tile, m-tile fastest

    // fragment read offsets (lane l: row l & 15 of a fragment, K chunks g and
    // g + 4 of the 128-byte block, g = l >> 4; swizzled chunk c ^ (row & 7))
    const int l15 = lane & 15, l7 = lane & 7, lg = lane >> 4;
    const uint32_t a_rd0 = (wm * 64 + l15) * 128 + ((lg ^ l7) << 4);
    const uint32_t a_rd1 = (wm * 64 + l15) * 128 + (((lg + 4) ^ l7) << 4);
    const uint32_t b_rd0 = SM::A_BYTES + (wn * WN + l15) * 128 + ((lg ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * WN + l15) * 128 + (((lg + 4) ^ l7) << 4);
    // A scales: the 16 bytes at slot wm*64 + 4*l15 hold rows wm*64 + mi*16 + l15
    // (mi = 0..3); B scales: natural order, 4 consecutive columns per read
    const uint32_t sa_rd = SM::A_BYTES + SM::B_BYTES + (wm * 64 + l15 * 4) * 4;
    // (P2: the scale of the B row whose K chunk the lane holds, column wn*WN + ni*16 + l15)
    const uint32_t sb_rd = SM::A_BYTES + SM::B_BYTES + SM::SA_BYTES + (wn * WN + (P2 ? l15 : 4 * lg)) * 4;
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
    // output: byte offset in the tile of the lane's first 16-byte store of
    // subtile mi after the regrouping in finish().  128-column tiles: row
    // wm*64 + mi*16 + l15, columns wn*WN + 8*lg .. +7.  256-column tiles (a
    // wave's row is one 128-byte line): row wm*64 + mi*16 + (l15 & ~1), bytes
    // 64*(l15 & 1) + 16*lg of the wave's 128; the second store is the next row.
    uint32_t o_off[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
        o_off[mi] = NI == 4 ? (uint32_t)(((wm * 64 + mi * 16 + (l15 & ~1)) * N + wn * WN) * 2 + 64 * (l15 & 1) + 16 * lg)
                            : (uint32_t)(((wm * 64 + mi * 16 + l15) * N + wn * WN) * 2 + 16 * lg);

    // DMA lane offset: swizzled chunk of row l/8 of a contiguous 1 KB segment
    // (8 rows of one token block); both operands share it
    const int lr = lane >> 3;
    const uint32_t seg_off = (uint32_t)(lr * WBK + (((lane & 7) ^ lr) << 4));
    // lane l < 16 of wave w fills A scale slot w*16 + l: row (w/4)*64 + (l%4)*16
    // + (w%4)*4 + l/4 (the slot layout above)
    const uint32_t sa_off = (uint32_t)(((wave >> 2) * 64 + (lane & 3) * 16 + (wave & 3) * 4 + ((lane & 15) >> 2)) * 4);
    const uint32_t sb_off = (uint32_t)((lane & (SROWS - 1)) * 4);

    // A tile is (j, s, f): the j-th expert with rows, then a slow and a fast
    // tile index.  The fast index runs over the smaller operand's tiles
    // (m-tiles when M <= N, else n-tiles), in groups of gf tiles, and the slow
    // index over the larger operand's tiles within a group: the 32 tiles one
    // XCD runs side by side cover a block of gf x 32/gf tiles, whose operand
    // tiles (about 1.2 MB at the training shape) stay in that XCD's L2 next
    // to the tiles' output stream.
    // Workgroup lb takes tiles lb, lb + G, ...; the step G is split into
    // carries so that no division runs per tile.
    struct Pos {
        int j, s, f;
    };
    const bool nfast = g.nfast != 0;
    const int ST0 = nfast ? MT : NT;
    const int FT = g.gf, ST = ((nfast ? NT : MT) / FT) * ST0;
    const int Gj = G / TPE, Gr = G - Gj * TPE, Gs = Gr / FT, Gf = Gr - Gs * FT;
    // (s, f) -> tile: s = group * ST0 + slow tile, fast tile = group * FT + f
    auto tile_of = [&](const Pos& p, int& mt, int& nt) {
        const int grp = p.s / ST0, sl = p.s - grp * ST0, fa = grp * FT + p.f;
        nt = nfast ? fa : sl;
        mt = nfast ? sl : fa;
    };
    auto step_pos = [&](Pos& p) {
        p.f += Gf;
        int c = p.f >= FT ? 1 : 0;
        p.f -= c * FT;
        p.s += Gs + c;
        c = p.s >= ST ? 1 : 0;
        p.s -= c * ST;
        p.j += Gj + c;
    };
    Pos p0;
    p0.j = lb / TPE;
    p0.s = (lb - p0.j * TPE) / FT;
    p0.f = lb - p0.j * TPE - p0.s * FT;
    auto nkb_of = [&](const Pos& p) -> int {
        return p.j < Lne ? (__builtin_amdgcn_readfirstlane(tab_x[p.j]) >> 10) : 0;
    };
    // The tiles an XCD runs side by side share one tile of the larger
    // operand; each starts its K loop at a different token block (its fast
    // index modulo the block count), so that they do not all request the same
    // lines of the shared tile at once.  Only the order of the fp32 block sums
    // changes.
    auto rot_of = [&](const Pos& p, int nkb) -> int { return nkb > 0 ? p.f % nkb : 0; };
    struct Src {
        const uint8_t* a;  // this wave's first A row at the segment start
        const uint8_t* b;
        const float* sa;   // the tile's A scales, first token block of the segment
        const float* sb;   // this wave's B scales, first token block
    };
    auto src_of = [&](const Pos& p) {
        int mt, nt;
        tile_of(p, mt, nt);
        const int64_t lo = __builtin_amdgcn_readfirstlane(tab_lo[p.j]);
        Src s;
        s.a = g.aT + ((lo / WBK) * M + (int64_t)mt * WBM + wave * ASEG * 8) * WBK;
        s.b = g.bT + ((lo / WBK) * N + (int64_t)nt * BN + wave * BSEG * 8) * WBK;
        s.sa = g.aT_s + (lo / WBK) * M + (int64_t)mt * WBM;
        s.sb = g.bT_s + (lo / WBK) * N + (int64_t)nt * BN + wave * SROWS;
        return s;
    };
    auto dst_of = [&](const Pos& p) -> uint16_t* {
        const int e = __builtin_amdgcn_readfirstlane(tab_x[p.j]) & 1023;
        int mt, nt;
        tile_of(p, mt, nt);
        return g.dW + (int64_t)e * M * N + (int64_t)mt * WBM * N + (int64_t)nt * BN;
    };

    // Waves 0-3 (one per SIMD) issue every stage's DMA: each moves its own
    // share and that of wave + 4 (A rows 4*ASEG*8 further, B rows 4*BSEG*8,
    // scales as the A rows), so waves 4-7 never stall on a DMA issue and keep
    // the matrix cores busy meanwhile.  Waves 4-7 issue no loads and so wait
    // for none: a stage is published by the barrier that follows the DMA
    // waves' own vmcnt wait.
    const bool dma_wave = wave < 4;
    auto issue = [&](auto stage_c, int kb, const Src& s) {
        constexpr int stage = decltype(stage_c)::value;
        if (!dma_wave) return;
        const uint32_t sA = sbase + (uint32_t)(stage * SM::STAGE);
        const uint32_t sB = sA + SM::A_BYTES;
        const uint32_t sSA = sB + SM::B_BYTES;
        const uint32_t sSB = sSA + SM::SA_BYTES;
        const uint8_t* a = s.a + (int64_t)kb * M * WBK;
        const uint8_t* b = s.b + (int64_t)kb * N * WBK;
        static_for<0, 2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;  // 0: own share, 1: wave + 4's
            const int w = wave + 4 * h;
#pragma unroll
            for (int i = 0; i < ASEG; ++i)
                dma16s(a + (h * 4 * ASEG * 8) * WBK + i * 1024, seg_off, sA + (w * ASEG + i) * 1024);
#pragma unroll
            for (int i = 0; i < BSEG; ++i)
                dma16s(b + (h * 4 * BSEG * 8) * WBK + i * 1024, seg_off, sB + (w * BSEG + i) * 1024);
            if (lane < 16) dma4s(s.sa + (int64_t)kb * M, sa_off + h * 64 * 4, sSA + w * 64);
            if (lane < SROWS) dma4s(s.sb + (int64_t)kb * N + h * 4 * SROWS, sb_off, sSB + w * SROWS * 4);
        });
    };

    // issue cursor: the K step two ahead of the one being waited for (i_kb
    // counts the tile's steps, i_kr is the token block it reads)
    Pos ip = p0;
    int i_kb = 0, i_nkb = nkb_of(ip), i_kr = rot_of(ip, i_nkb);
    Src isrc{};
    if (ip.j < Lne) isrc = src_of(ip);
    auto issue_next = [&](auto stage_c) -> bool {
        if (ip.j >= Lne) return false;
        issue(stage_c, i_kr, isrc);
        if (++i_kr == i_nkb) i_kr = 0;
        if (++i_kb == i_nkb) {
            step_pos(ip);
            i_kb = 0;
            i_nkb = nkb_of(ip);
            i_kr = rot_of(ip, i_nkb);
            if (ip.j < Lne) isrc = src_of(ip);
        }
        return true;
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    v4f acc[4][NI];
    v8i af[4], bfr[NI];
    float sa[4];  // A scales of the loaded block (rows of this lane)
    v4f sb[NI];   // B scales of the loaded block (4 columns per n-subtile)
    v4f ring[4];  // raw partials awaiting their rescale
    int ea[4], eb[NI];  // P2: E8M0 exponents of the lane's A rows and B rows
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) ea[mi] = 127;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) eb[ni] = 127;
    auto clear = [&]() {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;
            ring[mi] = zero4;
        }
    };
    clear();
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) sa[mi] = 0.f;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) sb[ni] = zero4;

    auto flush = [&]() {
        if constexpr (P2) return;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[mi][NI - 1] += ring[mi] * (sa[mi] * sb[NI - 1]);
    };
    auto load = [&](auto stage_c) {
        constexpr int st = decltype(stage_c)::value;
        pin(rA0[st]);
        pin(rA1[st]);
        pin(rB0[st]);
        pin(rB1[st]);
        pin(rSA[st]);
        pin(rSB[st]);
        const uint32_t pa0 = rA0[st], pa1 = rA1[st], pb0 = rB0[st], pb1 = rB1[st];
        const uint32_t psa = rSA[st], psb = rSB[st];
        const u32x4 sa4 = lds16<0>(psa);
        u32x4 sbn[NI];
        uint32_t sb1[NI];
        static_for<0, NI>([&](auto nc) {
            constexpr int ni = decltype(nc)::value;
            if constexpr (P2)
                sb1[ni] = lds4<ni * 64>(psb);
            else
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
        if constexpr (P2) {
            // positive powers of two: the E8M0 code is the exponent field
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) ea[mi] = (int)(sav[mi] >> 23);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) eb[ni] = (int)(sb1[ni] >> 23);
        } else {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) sa[mi] = __uint_as_float(sav[mi]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) sb[ni] = __builtin_bit_cast(v4f, sbn[ni]);
        }
        wait_lgkm0();
    };
    auto compute = [&]() {
        if constexpr (P2) {
            static_for<0, 4 * NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int ni = j / 4, mi = j % 4;
                acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], af[mi], acc[mi][ni], eb[ni], ea[mi]);
            });
            return;
        }
        static_for<0, 4 * NI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int ni = j / 4, mi = j % 4;
            if constexpr (j >= 4) acc[mi][ni - 1] += ring[mi] * (sa[mi] * sb[ni - 1]);
            ring[mi] = mfma16x16x128(bfr[ni], af[mi]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // finished tile: bf16 straight from the accumulators, then they restart.
    // Lane (l15, lg) holds columns 16c + 4lg .. +3 of n-subtile c: 4-column
    // chunk q = 4c + lg of the wave's row.  Exchanging the chunk-slot bit c0
    // with lane-group bit 1 (swap32) and then with lane-group bit 0 (swap16)
    // leaves slot 2h + s holding chunk 8h + 2lg + s: 8 consecutive columns per
    // lane for each h, piece P_h = bytes 64h + 16lg of row l15.
    // 256-column tiles: a store that fills whole 128-byte lines moves about
    // 1.5x the bytes per clock of one that writes half lines (measured, 8 rows
    // x 128 B against 16 rows x 64 B per instruction), so the lanes of rows 2u
    // and 2u + 1 trade pieces (DPP quad permute [1, 0, 3, 2]): the even lane
    // passes P_1 and takes its partner's P_0, the odd lane the reverse.  Store
    // 0 then writes row 2u whole (P_0 from the even lanes, P_1 from the odd
    // ones), store 1 row 2u + 1.
    const bool odd_row = (lane & 1) != 0;
    auto finish = [&](uint16_t* dst) {
        flush();
        uint8_t* d = reinterpret_cast<uint8_t*>(dst);
        static_for<0, 4>([&](auto ic) {
            constexpr int mi = decltype(ic)::value;
            uint32_t x[NI], y[NI];  // columns (0, 1) and (2, 3) of each chunk, packed bf16
#pragma unroll
            for (int c = 0; c < NI; ++c) {
                const v4f a = acc[mi][c];
                x[c] = cvt_bf16x2(a.x, a.y);
                y[c] = cvt_bf16x2(a.z, a.w);
            }
#pragma unroll
            for (int c = 0; c < NI; c += 2) {
                swap32(x[c], x[c + 1]);
                swap32(y[c], y[c + 1]);
                swap16(x[c], x[c + 1]);
                swap16(y[c], y[c + 1]);
            }
            if constexpr (NI == 4) {
                const u32x4 p0 = {x[0], y[0], x[1], y[1]}, p1 = {x[2], y[2], x[3], y[3]};
                const u32x4 snd = odd_row ? p0 : p1;
                u32x4 r;
#pragma unroll
                for (int c = 0; c < 4; ++c) r[c] = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd[c], 0xB1, 0xF, 0xF, false);
                st_stream(reinterpret_cast<u32x4*>(d + o_off[mi]), odd_row ? r : p0);
                st_stream(reinterpret_cast<u32x4*>(d + o_off[mi] + 2 * N), odd_row ? p1 : r);
            } else {
                st_stream(reinterpret_cast<u32x4*>(d + o_off[mi]), u32x4{x[0], y[0], x[1], y[1]});
            }
        });
        clear();
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    if (lb < total) {
        issue_next(S0{});
        // vector-memory ops issued after the stage the next step waits for:
        // stores two steps back, the next stage's loads, stores one step back
        // (a DMA wave issues 2 * NLD loads per stage, the others none)
        constexpr int NLD2 = 2 * NLD;
        int yng = issue_next(S1{}) ? NLD2 : 0;
        int ns1 = 0;  // NST if the previous step issued stores
        auto wait_stage = [&]() {
            if (!dma_wave) return;
            if (yng == NLD2) wait_vmcnt<NLD2>();  // no stores in flight: the common case
            else wait_younger<NLD2, NST>(yng);
        };
        auto account = [&](bool iss, bool sto) {
            yng = ns1 + (iss ? NLD2 : 0) + (sto ? NST : 0);
            ns1 = sto ? NST : 0;
        };
        Pos cp = p0;  // tile of the block being computed
        int c_kb = 0, c_nkb = nkb_of(cp);

        if (wave < 4) {
            // group 0: wait, issue, load, | compute (and store a finished tile)
            auto step = [&](auto st_c) -> bool {
                constexpr int st = decltype(st_c)::value;
                wait_stage();
                phase_barrier();
                const bool iss = issue_next(std::integral_constant<int, (st + 2) % 3>{});
                load(st_c);
                phase_barrier();
                compute();
                const bool sto = ++c_kb == c_nkb;
                account(iss, sto);
                if (sto) {
                    finish(dst_of(cp));
                    step_pos(cp);
                    c_kb = 0;
                    if (cp.j >= Lne) return false;
                    c_nkb = nkb_of(cp);
                }
                return true;
            };
            // one exit: the live-out fragments and accumulators keep their
            // registers (break exits after every step made the allocator spill)
            bool more = true;
            while (more) {
                more = step(S0{});
                if (more) more = step(S1{});
                if (more) more = step(S2{});
            }
        } else {
            // group 1, half a step behind: wait, issue, compute the previous
            // block (and store a finished tile), | load
            Pos lp = p0;  // tile of the block being loaded
            int l_kb = 0, l_nkb = c_nkb;
            auto step = [&](auto st_c, bool prev) -> bool {
                constexpr int st = decltype(st_c)::value;
                wait_stage();
                phase_barrier();
                const bool iss = issue_next(std::integral_constant<int, (st + 2) % 3>{});
                bool sto = false;
                if (prev) {
                    compute();
                    sto = ++c_kb == c_nkb;
                    if (sto) {
                        finish(dst_of(cp));
                        step_pos(cp);
                        c_kb = 0;
                        c_nkb = nkb_of(cp);
                    }
                }
                account(iss, sto);
                phase_barrier();
                load(st_c);
                if (++l_kb == l_nkb) {
                    step_pos(lp);
                    l_kb = 0;
                    if (lp.j >= Lne) return false;
                    l_nkb = nkb_of(lp);
                }
                return true;
            };
            bool more = step(S0{}, false);
            while (more) {
                more = step(S1{}, true);
                if (more) more = step(S2{}, true);
                if (more) more = step(S0{}, true);
            }
            compute();  // the last block, loaded by the last step
            finish(dst_of(cp));
        }
    }

    zero_fill_empty(g, tid);
}


// ---------------------------------------------------------------- A resident
//
// 128 x 256 tiles for experts with at most ARES_KB token blocks (fp32
// scales, or P2: the E8M0 exponents applied by the block-scaled MFMA).  A
// unit of work is (expert, m-tile): the unit's A operand, all of the
// expert's token blocks (16 KB of codes and 512 B of row scales each), is
// moved into LDS once and stays there while the unit sweeps its n-tiles; only
// B streams, through a two-stage ring of 33 KB stages.  A K step then moves
// 32 KB instead of 48, and the 32 workgroups of an XCD, running m-tiles of
// one expert, read the same B tiles at about the same time.  The K step, the
// ping-pong groups, the epilogue and the waits are those of wgrad_fp8_kernel
// with a ring two stages deep (the DMA of a step goes out one step ahead).
// At the first step of a unit both groups wait at one more barrier while the
// DMA waves replace the A region: every read of the old one ends before the
// step's first barrier.
constexpr int ARES_KB = 5;
struct AresSmem {
    static constexpr int A_BLK = WBM * WBK;       // 16 KB of codes per token block
    static constexpr int SA_BLK = WBM * 4;        // its 128 row scales
    static constexpr int SA0 = ARES_KB * A_BLK;   // the scales follow the codes
    static constexpr int RING = SA0 + ARES_KB * SA_BLK;
    static constexpr int B_BYTES = 256 * WBK;
    static constexpr int SB_BYTES = 256 * 4;
    static constexpr int STAGE = B_BYTES + SB_BYTES;
    static constexpr int TAB = RING + 2 * STAGE;  // experts: count, packed id|nkb, lo
    static constexpr int TOTAL = TAB + (1 + 2 * WMAXL) * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS");
};

template <bool P2>
__global__ __launch_bounds__(WTHREADS, 1) void wgrad_ares_kernel(WgradArgs g) {
    using SM = AresSmem;
    constexpr int BN = 256, WN = 64, NI = 4;
    constexpr int ASEG = WBM / 64;   // 1 KB A segments per wave share and block
    constexpr int BSEG = BN / 64;    // 1 KB B segments per wave share and stage
    constexpr int SROWS = BN / 8;    // B scales per wave share
    constexpr int NLD2 = 2 * (BSEG + 1);  // B DMA instructions of a DMA wave per stage
    constexpr int NST = 2 * NI;      // 16-byte stores per wave per tile
    static_assert(NLD2 + NST < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    int* const tab = reinterpret_cast<int*>(smem + SM::TAB);
    int* const tab_x = tab + 1;           // e | nkb << 10
    int* const tab_lo = tab + 1 + WMAXL;  // first row of the segment

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t rcap = g.row_cap;
    const int M = g.M, N = g.N;
    const int MT = M / WBM, NT = N / BN;
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    build_expert_table(g, rcap, wave, lane, tab, tab_x, tab_lo);
    __syncthreads();
    const int Lne = __builtin_amdgcn_readfirstlane(tab[0]);
    const int units = Lne * MT;  // (expert, m-tile), expert-major

    // fragment reads (lane l: row l & 15 of a fragment, K chunks g and g + 4
    // of the 128-byte block, g = l >> 4; swizzled chunk c ^ (row & 7)); A from
    // block kr of the resident region, B from a ring stage
    const int l15 = lane & 15, l7 = lane & 7, lg = lane >> 4;
    const uint32_t a_rd0 = sbase + (wm * 64 + l15) * 128 + ((lg ^ l7) << 4);
    const uint32_t a_rd1 = sbase + (wm * 64 + l15) * 128 + (((lg + 4) ^ l7) << 4);
    // A scales: the 16 bytes at slot wm*64 + 4*l15 of a block hold rows
    // wm*64 + mi*16 + l15 (mi = 0..3); B scales: 4 consecutive columns per read
    const uint32_t sa_rd = sbase + SM::SA0 + (wm * 64 + l15 * 4) * 4;
    uint32_t rB0[2], rB1[2], rSB[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const uint32_t b = sbase + SM::RING + (uint32_t)(st * SM::STAGE);
        rB0[st] = b + (wn * WN + l15) * 128 + ((lg ^ l7) << 4);
        rB1[st] = b + (wn * WN + l15) * 128 + (((lg + 4) ^ l7) << 4);
        // (P2: the scale of the B row whose K chunk the lane holds)
        rSB[st] = b + SM::B_BYTES + (wn * WN + (P2 ? l15 : 4 * lg)) * 4;
    }
    // output: the lane's first 16-byte store of subtile mi (whole 128-byte
    // lines, as in wgrad_fp8_kernel): row wm*64 + mi*16 + (l15 & ~1), bytes
    // 64*(l15 & 1) + 16*lg of the wave's 128; the second store is the next row
    uint32_t o_off[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
        o_off[mi] = (uint32_t)(((wm * 64 + mi * 16 + (l15 & ~1)) * N + wn * WN) * 2 + 64 * (l15 & 1) + 16 * lg);
    const int lr = lane >> 3;
    const uint32_t seg_off = (uint32_t)(lr * WBK + (((lane & 7) ^ lr) << 4));
    const uint32_t sa_off = (uint32_t)(((wave >> 2) * 64 + (lane & 3) * 16 + (wave & 3) * 4 + ((lane & 15) >> 2)) * 4);
    const uint32_t sb_off = (uint32_t)((lane & (SROWS - 1)) * 4);

    // step cursor: unit u (this workgroup's units are lb, lb + G, ...), n-tile
    // nt, step i of the tile's K loop; the K loop starts at block rot = m-tile
    // mod nkb, so that the m-tiles an XCD runs side by side do not request
    // the same lines of their shared B tile at once (only the order of the
    // fp32 block sums changes)
    struct Cur {
        int u, nt, i, nkb, rot, mt;
        int64_t blk0;  // first token block of the expert's segment
        int e;
    };
    // (the divisions run once per unit; their results are wave-uniform and
    // kept in scalar registers)
    auto unit_at = [&](Cur& c, int u) {
        c.u = u;
        c.nt = 0;
        c.i = 0;
        if (u >= units) return;
        const int j = __builtin_amdgcn_readfirstlane(u / MT);
        c.mt = __builtin_amdgcn_readfirstlane(u - j * MT);
        const int x = __builtin_amdgcn_readfirstlane(tab_x[j]);
        c.e = x & 1023;
        c.nkb = x >> 10;
        c.rot = __builtin_amdgcn_readfirstlane(c.mt % c.nkb);
        c.blk0 = __builtin_amdgcn_readfirstlane(tab_lo[j]) / WBK;
    };
    // advance one K step; true when the step entered a new unit
    auto advance = [&](Cur& c) -> bool {
        if (++c.i < c.nkb) return false;
        c.i = 0;
        if (++c.nt < NT) return false;
        unit_at(c, c.u + G);
        return true;
    };
    auto kr_of = [&](const Cur& c) { int k = c.i + c.rot; return k >= c.nkb ? k - c.nkb : k; };

    const bool dma_wave = wave < 4;
    // the unit's A blocks into the resident region (DMA waves: their own share
    // and that of wave + 4, as in wgrad_fp8_kernel)
    auto issue_a = [&](const Cur& c) {
        if (!dma_wave) return;
        const uint8_t* a = g.aT + ((c.blk0 * M + (int64_t)c.mt * WBM + wave * ASEG * 8) * WBK);
        const float* sa = g.aT_s + c.blk0 * M + (int64_t)c.mt * WBM;
        for (int kb = 0; kb < c.nkb; ++kb) {
            const uint32_t sA = sbase + (uint32_t)(kb * SM::A_BLK), sSA = sbase + SM::SA0 + (uint32_t)(kb * SM::SA_BLK);
            static_for<0, 2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
                const int w = wave + 4 * h;
#pragma unroll
                for (int i = 0; i < ASEG; ++i)
                    dma16s(a + (int64_t)kb * M * WBK + (h * 4 * ASEG * 8) * WBK + i * 1024, seg_off,
                           sA + (w * ASEG + i) * 1024);
                if (lane < 16) dma4s(sa + (int64_t)kb * M, sa_off + h * 64 * 4, sSA + w * 64);
            });
        }
    };
    // B block kr of (unit, n-tile) into ring stage st
    auto issue_b = [&](int st, const Cur& c) {
        if (!dma_wave) return;
        const int kr = kr_of(c);
        const uint8_t* b = g.bT + (((c.blk0 + kr) * N + (int64_t)c.nt * BN + wave * BSEG * 8) * WBK);
        const float* sb = g.bT_s + (c.blk0 + kr) * N + (int64_t)c.nt * BN + wave * SROWS;
        const uint32_t sB = sbase + SM::RING + (uint32_t)(st * SM::STAGE), sSB = sB + SM::B_BYTES;
        static_for<0, 2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const int w = wave + 4 * h;
#pragma unroll
            for (int i = 0; i < BSEG; ++i)
                dma16s(b + (h * 4 * BSEG * 8) * WBK + i * 1024, seg_off, sB + (w * BSEG + i) * 1024);
            if (lane < SROWS) dma4s(sb + h * 4 * SROWS, sb_off, sSB + w * SROWS * 4);
        });
    };
    auto dst_of = [&](const Cur& c) -> uint16_t* {
        return g.dW + (int64_t)c.e * M * N + (int64_t)c.mt * WBM * N + (int64_t)c.nt * BN;
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    v4f acc[4][NI];
    v8i af[4], bfr[NI];
    float sa[4];  // A scales of the loaded block (rows of this lane)
    v4f sb[NI];   // B scales of the loaded block (4 columns per n-subtile)
    v4f ring[4];  // raw partials awaiting their rescale
    int ea[4], eb[NI];  // P2: E8M0 exponents of the lane's A rows and B rows
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) ea[mi] = 127;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) eb[ni] = 127;
    auto clear = [&]() {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;
            ring[mi] = zero4;
        }
    };
    clear();
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) sa[mi] = 0.f;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) sb[ni] = zero4;
    auto flush = [&]() {
        if constexpr (P2) return;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[mi][NI - 1] += ring[mi] * (sa[mi] * sb[NI - 1]);
    };
    auto load = [&](auto st_c, int kr) {
        constexpr int st = decltype(st_c)::value;
        uint32_t pa0 = a_rd0 + (uint32_t)(kr * SM::A_BLK), pa1 = a_rd1 + (uint32_t)(kr * SM::A_BLK);
        uint32_t psa = sa_rd + (uint32_t)(kr * SM::SA_BLK);
        pin(pa0);
        pin(pa1);
        pin(psa);
        pin(rB0[st]);
        pin(rB1[st]);
        pin(rSB[st]);
        const uint32_t pb0 = rB0[st], pb1 = rB1[st], psb = rSB[st];
        const u32x4 sa4 = lds16<0>(psa);
        u32x4 sbn[NI];
        uint32_t sb1[NI];
        static_for<0, NI>([&](auto nc) {
            constexpr int ni = decltype(nc)::value;
            if constexpr (P2)
                sb1[ni] = lds4<ni * 64>(psb);
            else
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
        if constexpr (P2) {
            // positive powers of two: the E8M0 code is the exponent field
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) ea[mi] = (int)(sav[mi] >> 23);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) eb[ni] = (int)(sb1[ni] >> 23);
        } else {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) sa[mi] = __uint_as_float(sav[mi]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) sb[ni] = __builtin_bit_cast(v4f, sbn[ni]);
        }
        wait_lgkm0();
    };
    auto compute = [&]() {
        if constexpr (P2) {
            static_for<0, 4 * NI>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                constexpr int ni = j / 4, mi = j % 4;
                acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], af[mi], acc[mi][ni], eb[ni], ea[mi]);
            });
            return;
        }
        static_for<0, 4 * NI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int ni = j / 4, mi = j % 4;
            if constexpr (j >= 4) acc[mi][ni - 1] += ring[mi] * (sa[mi] * sb[ni - 1]);
            ring[mi] = mfma16x16x128(bfr[ni], af[mi]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    const bool odd_row = (lane & 1) != 0;
    auto finish = [&](uint16_t* dst) {
        flush();
        uint8_t* d = reinterpret_cast<uint8_t*>(dst);
        static_for<0, 4>([&](auto ic) {
            constexpr int mi = decltype(ic)::value;
            uint32_t x[NI], y[NI];
#pragma unroll
            for (int c = 0; c < NI; ++c) {
                const v4f a = acc[mi][c];
                x[c] = cvt_bf16x2(a.x, a.y);
                y[c] = cvt_bf16x2(a.z, a.w);
            }
#pragma unroll
            for (int c = 0; c < NI; c += 2) {
                swap32(x[c], x[c + 1]);
                swap32(y[c], y[c + 1]);
                swap16(x[c], x[c + 1]);
                swap16(y[c], y[c + 1]);
            }
            const u32x4 p0 = {x[0], y[0], x[1], y[1]}, p1 = {x[2], y[2], x[3], y[3]};
            const u32x4 snd = odd_row ? p0 : p1;
            u32x4 r;
#pragma unroll
            for (int c = 0; c < 4; ++c) r[c] = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd[c], 0xB1, 0xF, 0xF, false);
            st_stream(reinterpret_cast<u32x4*>(d + o_off[mi]), odd_row ? r : p0);
            st_stream(reinterpret_cast<u32x4*>(d + o_off[mi] + 2 * N), odd_row ? p1 : r);
        });
        clear();
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    Cur ic;  // issue cursor: the step after the one being loaded
    unit_at(ic, lb);
    if (ic.u < units) {
        // prologue: the first unit's A and step 0's B (stage 0)
        issue_a(ic);
        issue_b(0, ic);
        advance(ic);
        // DMA waves: stores issued after the B DMA the next wait is for
        // (group 0: its finish one step back)
        int yng = 0;
        auto wait_stage = [&]() {
            if (!dma_wave) return;
            if (yng == 0) wait_vmcnt<0>();
            else wait_vmcnt<NST>();
        };
        // the B of the next step goes out (DMA waves), into stage st
        auto issue_next = [&](int st) -> bool {
            if (ic.u >= units) return false;
            issue_b(st, ic);
            advance(ic);
            return true;
        };
        Cur lc;  // the step being loaded
        unit_at(lc, lb);
        Cur cc = lc;  // the step being computed
        // one step; false after the last one
        if (wave < 4) {
            // group 0: wait, (A of a new unit,) issue, load | compute (and store a finished tile)
            auto step = [&](auto st_c, bool sw) -> bool {
                constexpr int st = decltype(st_c)::value;
                wait_stage();
                phase_barrier();
                if (sw) {
                    issue_a(lc);
                    wait_vmcnt<0>();
                    phase_barrier();
                }
                issue_next(st ^ 1);
                load(st_c, kr_of(lc));
                phase_barrier();
                compute();
                const bool last_k = cc.i + 1 == cc.nkb;
                uint16_t* dst = dst_of(cc);
                advance(cc);
                yng = 0;
                if (last_k) {
                    finish(dst);
                    yng = NST;
                }
                return cc.u < units;
            };
            bool more = true, sw = false;
            while (more) {
                more = step(S0{}, sw);
                sw = advance(lc);
                if (more) {
                    more = step(S1{}, sw);
                    sw = advance(lc);
                }
            }
        } else {
            // group 1, half a step behind: (A of a new unit,) compute the
            // previous block (and store a finished tile) | load
            // (one loop exit: the live-out fragments and accumulators keep
            // their registers)
            bool sw = false;
            auto step = [&](auto st_c, auto prev_c) -> bool {
                phase_barrier();
                if (sw) phase_barrier();
                if constexpr (decltype(prev_c)::value) {
                    compute();
                    const bool last_k = cc.i + 1 == cc.nkb;
                    uint16_t* dst = dst_of(cc);
                    advance(cc);
                    if (last_k) finish(dst);
                }
                phase_barrier();
                load(st_c, kr_of(lc));
                sw = advance(lc);
                return lc.u < units;
            };
            using NoPrev = std::false_type;
            using Prev = std::true_type;
            bool more = step(S0{}, NoPrev{});
            while (more) {
                more = step(S1{}, Prev{});
                if (more) more = step(S0{}, Prev{});
            }
            compute();  // the last block, loaded by the last step
            finish(dst_of(cc));
        }
    }
    zero_fill_empty(g, tid);
}


// ---------------------------------------------------------------- 256 x 256 tiles
//
// The same products with power-of-two scales on 256 x 256 tiles (M and N
// multiples of 256).  A K step moves 64 KB of operands (a token block's 256 A
// rows and 256 B rows, each a contiguous 32 KB piece) for twice the MFMA work
// of a 128 x 256 tile's 48 KB.  The K step is the forward grouped GEMM's
// 256 x 256 one: 8 waves as 2 (M) x 4 (N) of 128 x 64, eight 16-row subtiles
// streamed from LDS while the wave's four B fragments stay in registers, two
// 66 KB stages, and one barrier per step before its last subtile that both
// frees the stage just read and publishes the next.  The per-row scales of
// both operands are E8M0 exponents the block-scaled MFMA applies.  Waves 0-3
// issue all DMA (their own share and that of wave + 4); the next tile's first
// step is issued before the epilogue stores, and the waits that follow count
// those stores instead of draining them.
// With fp32 scales the factor sA[m] * sB[n] of every partial costs eight VALU
// operations per MFMA (four column scales per lane), as long as the MFMA
// itself; at this tile size the registers for them do not fit next to the
// accumulators without spilling, and the 128 x 256 kernel above (the same
// speed then, measured) takes those products.
struct WideWgradSmem {
    static constexpr int A_BYTES = 256 * WBK;
    static constexpr int B_BYTES = 256 * WBK;
    static constexpr int SA_BYTES = 256 * 4;
    static constexpr int SB_BYTES = 256 * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int TAB = 2 * STAGE;  // experts with rows: count, packed id|nkb, lo
    static constexpr int TOTAL = TAB + (1 + 2 * WMAXL) * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS");
};

__global__ __launch_bounds__(WTHREADS, 1) void wgrad_wide_kernel(WgradArgs g) {
    using SM = WideWgradSmem;
    constexpr int MI = 8, NI = 4;  // 16 x 16 subtiles of a wave's 128 x 64
    constexpr int NST = 2 * MI;    // 16-byte stores per wave per tile

    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];
    int* const tab = reinterpret_cast<int*>(smem + SM::TAB);
    int* const tab_x = tab + 1;           // e | nkb << 10
    int* const tab_lo = tab + 1 + WMAXL;  // first row of the segment

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t rcap = g.row_cap;
    const int M = g.M, N = g.N;
    const int MT = M / 256, NT = N / 256, TPE = MT * NT;
    const int G = gridDim.x;
    const int lb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));

    // experts of this launch (token block counts kb_min..kb_max), in order
    build_expert_table(g, rcap, wave, lane, tab, tab_x, tab_lo);
    __syncthreads();
    const int Lne = __builtin_amdgcn_readfirstlane(tab[0]);

    // tile order (j, s, f) as in wgrad_fp8_kernel: the fast index runs over
    // the smaller operand's tiles
    struct Pos {
        int j, s, f;
    };
    const bool nfast = g.nfast != 0;
    const int ST0 = nfast ? MT : NT;
    const int FT = g.gf, ST = ((nfast ? NT : MT) / FT) * ST0;
    const int Gj = G / TPE, Gr = G - Gj * TPE, Gs = Gr / FT, Gf = Gr - Gs * FT;
    // (s, f) -> tile: s = group * ST0 + slow tile, fast tile = group * FT + f
    auto tile_of = [&](const Pos& p, int& mt, int& nt) {
        const int grp = p.s / ST0, sl = p.s - grp * ST0, fa = grp * FT + p.f;
        nt = nfast ? fa : sl;
        mt = nfast ? sl : fa;
    };
    auto step_pos = [&](Pos& p) {
        p.f += Gf;
        int c = p.f >= FT ? 1 : 0;
        p.f -= c * FT;
        p.s += Gs + c;
        c = p.s >= ST ? 1 : 0;
        p.s -= c * ST;
        p.j += Gj + c;
    };
    Pos cp;
    cp.j = lb / TPE;
    cp.s = (lb - cp.j * TPE) / FT;
    cp.f = lb - cp.j * TPE - cp.s * FT;

    // fragment reads (stage-relative): lane l holds row l & 15 of a 16-row
    // fragment, K chunks c0 and c0 + 4 (c0 = l >> 4) of the 128-byte block,
    // stored at chunk c ^ (row & 7)
    const int l15 = lane & 15, l7 = lane & 7, c0 = lane >> 4;
    const uint32_t a_rd0 = (wm * 128 + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t a_rd1 = (wm * 128 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    const uint32_t b_rd0 = SM::A_BYTES + (wn * 64 + l15) * 128 + ((c0 ^ l7) << 4);
    const uint32_t b_rd1 = SM::A_BYTES + (wn * 64 + l15) * 128 + (((c0 + 4) ^ l7) << 4);
    // scales: the A row and the B row whose K chunk the lane holds, rows
    // wm*128 + mi*16 + l15 and wn*64 + ni*16 + l15 (64 bytes apart per subtile)
    const uint32_t sa_rd = SM::A_BYTES + SM::B_BYTES + (wm * 128 + l15) * 4;
    const uint32_t sb_rd = SM::A_BYTES + SM::B_BYTES + SM::SA_BYTES + (wn * 64 + l15) * 4;

    // DMA: a 1 KB segment is 8 rows of one token block; lane l moves chunk
    // (l & 7) ^ (l >> 3) of row l >> 3 to LDS byte l * 16 (the swizzle above).
    // The lane offsets are formed where a step is issued (not held in
    // registers across the K loop).
    auto seg_off_of = [&]() {
        const uint32_t l = (uint32_t)__lane_id();
        return ((l >> 3) * WBK) | ((((l & 7) ^ (l >> 3))) << 4);
    };
    // epilogue: byte offset in the tile of the lane's first store of a 16-row
    // subtile after the regrouping: row wm*128 + (l15 & ~1), bytes
    // 64*(l15 & 1) + 16*c0 of the wave's 128 (its second store is the next
    // row; each 16-row subtile is 16*N*2 further)
    const uint32_t o_lane0 = (uint32_t)(((wm * 128 + (l15 & ~1)) * N + wn * 64) * 2 + 64 * (l15 & 1) + 16 * c0);
    const bool odd_row = (l15 & 1) != 0;

    struct Src {
        const uint8_t* a;  // the tile's first A row, first token block of the segment
        const uint8_t* b;
        const float* sa;
        const float* sb;
        int nkb;
        int rot;  // first token block of the K loop
    };
    // The tiles an XCD runs side by side share one tile of the larger operand;
    // each starts its K loop at a different token block (its fast index
    // modulo the block count), so that they do not all request the same
    // lines of the shared tile at once (queueing on the same L2 channels).
    // Only the order of the fp32 block sums changes.
    auto src_of = [&](const Pos& p) {
        int mt, nt;
        tile_of(p, mt, nt);
        const int x = __builtin_amdgcn_readfirstlane(tab_x[p.j]);
        const int64_t blk0 = __builtin_amdgcn_readfirstlane(tab_lo[p.j]) / WBK;
        Src s;
        s.a = g.aT + (blk0 * M + (int64_t)mt * 256) * WBK;
        s.b = g.bT + (blk0 * N + (int64_t)nt * 256) * WBK;
        s.sa = g.aT_s + blk0 * M + (int64_t)mt * 256;
        s.sb = g.bT_s + blk0 * N + (int64_t)nt * 256;
        s.nkb = x >> 10;
        s.rot = p.f % s.nkb;
        return s;
    };
    auto dst_of = [&](const Pos& p) -> uint16_t* {
        int mt, nt;
        tile_of(p, mt, nt);
        const int e = __builtin_amdgcn_readfirstlane(tab_x[p.j]) & 1023;
        return g.dW + (int64_t)e * M * N + (int64_t)mt * 256 * N + (int64_t)nt * 256;
    };

    const bool dma_wave = wave < 4;
    // step kb of a tile into the stage at LDS address sA
    auto issue = [&](uint32_t sA, int kb, const Src& sr) {
        if (!dma_wave) return;
        const uint32_t sB = sA + SM::A_BYTES;
        kb += sr.rot;
        if (kb >= sr.nkb) kb -= sr.nkb;
        const uint8_t* a = sr.a + (int64_t)kb * M * WBK;
        const uint8_t* b = sr.b + (int64_t)kb * N * WBK;
        const uint32_t seg_off = seg_off_of();
        const uint32_t s16_off = (uint32_t)__lane_id() * 16;
        static_for<0, 2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const int w = wave + 4 * h;
#pragma unroll
            for (int i = 0; i < 4; ++i) dma16s(a + (w * 32 + 8 * i) * WBK, seg_off, sA + (w * 4 + i) * 1024);
#pragma unroll
            for (int i = 0; i < 4; ++i) dma16s(b + (w * 32 + 8 * i) * WBK, seg_off, sB + (w * 4 + i) * 1024);
        });
        if (wave == 0) dma16s(sr.sa + (int64_t)kb * M, s16_off, sB + SM::B_BYTES);
        if (wave == 1) dma16s(sr.sb + (int64_t)kb * N, s16_off, sB + SM::B_BYTES + SM::SA_BYTES);
    };
    auto lds_barrier = [&]() {
        wait_lgkm0();
        phase_barrier();
    };

    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    v4f acc[MI][NI];
    v8i bfr[NI];
    int eb[NI];        // E8M0 exponents of the lane's B rows
    v8i afc;           // the current subtile's A fragment ...
    uint32_t sac;      // ... and the A scale of its row (bits), read one subtile ahead
    auto read_b = [&](auto nc, uint32_t pb0, uint32_t pb1) {
        constexpr int ni = decltype(nc)::value;
        bfr[ni] = join8(lds16<ni * 2048>(pb0), lds16<ni * 2048>(pb1));
    };
    auto read_a = [&](auto mc, uint32_t pa0, uint32_t pa1) {
        constexpr int mi = decltype(mc)::value;
        return join8(lds16<mi * 2048>(pa0), lds16<mi * 2048>(pa1));
    };
    auto read_sa = [&](auto mc, uint32_t psa) {
        constexpr int mi = decltype(mc)::value;
        return lds4<mi * 64>(psa);
    };
    // positive powers of two: the E8M0 code is the fp32 exponent field
    auto read_sb = [&](uint32_t psb) {
        static_for<0, NI>([&](auto nc) {
            constexpr int ni = decltype(nc)::value;
            eb[ni] = (int)(lds4<ni * 64>(psb) >> 23);
        });
    };
    // every operand of a step, from the stage at LDS address sX
    auto read_step = [&](uint32_t sX) {
        pin_s(sX);
        uint32_t pb0 = sX + b_rd0, pb1 = sX + b_rd1, psa = sX + sa_rd, psb = sX + sb_rd;
        uint32_t pa0 = sX + a_rd0, pa1 = sX + a_rd1;
        pin(pb0); pin(pb1); pin(psa); pin(psb); pin(pa0); pin(pa1);
        static_for<0, NI>([&](auto nc) { read_b(nc, pb0, pb1); });
        read_sb(psb);
        afc = read_a(std::integral_constant<int, 0>{}, pa0, pa1);
        sac = read_sa(std::integral_constant<int, 0>{}, psa);
    };
    // four MFMAs of subtile mi, the scales applied by the matrix core
    auto subtile = [&](auto mc, const v8i& af, uint32_t sab) {
        const int ea = (int)(sab >> 23);
        static_for<0, NI>([&](auto nc) {
            constexpr int ni = decltype(nc)::value;
            acc[decltype(mc)::value][ni] = mfma16x16x128_e8m0(bfr[ni], af, acc[decltype(mc)::value][ni], eb[ni], ea);
        });
    };

    // stores issued after the DMA of the step the next wait is for (the
    // previous tile's epilogue), so that the wait does not drain them
    bool stores_out = false;
    Src cs{};
    bool have = cp.j < Lne;
    if (have) {
        cs = src_of(cp);
        issue(sbase, 0, cs);
    }
    while (have) {
        const int nkb = cs.nkb;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = zero4;

        // one K step from stage st; see gemm_wide_kernel for the schedule
        auto kstep = [&](auto st_c, int kb) {
            constexpr int st = decltype(st_c)::value;
            uint32_t sA = sbase + (uint32_t)(st * SM::STAGE);
            uint32_t sN = sbase + (uint32_t)((st ^ 1) * SM::STAGE);
            pin_s(sA);
            pin_s(sN);
            {
                uint32_t pa0 = sA + a_rd0, pa1 = sA + a_rd1, psa = sA + sa_rd;
                pin(pa0); pin(pa1); pin(psa);
                static_for<0, MI - 1>([&](auto mc) {
                    constexpr int mi = decltype(mc)::value;
                    const v8i afn = read_a(std::integral_constant<int, mi + 1>{}, pa0, pa1);
                    const uint32_t san = read_sa(std::integral_constant<int, mi + 1>{}, psa);
                    subtile(mc, afc, sac);
                    __builtin_amdgcn_sched_barrier(0);
                    afc = afn;
                    sac = san;
                });
            }
            // step kb + 1 has landed (the stores of the previous tile's
            // epilogue, a step older, with it)
            wait_vmcnt<0>();
            lds_barrier();
            if (kb + 2 < nkb) issue(sA, kb + 2, cs);
            {
                uint32_t pb0 = sN + b_rd0, pb1 = sN + b_rd1;
                pin(pb0); pin(pb1);
                constexpr int mi = MI - 1;
                const int ea = (int)(sac >> 23);
                static_for<0, NI>([&](auto nc) {
                    constexpr int ni = decltype(nc)::value;
                    acc[mi][ni] = mfma16x16x128_e8m0(bfr[ni], afc, acc[mi][ni], eb[ni], ea);
                    read_b(nc, pb0, pb1);
                    __builtin_amdgcn_sched_barrier(0);
                });
                // the next step's scales and first A fragment (unused values
                // after a tile's last step)
                uint32_t psa = sN + sa_rd, psb = sN + sb_rd, pa0 = sN + a_rd0, pa1 = sN + a_rd1;
                pin(psa); pin(psb); pin(pa0); pin(pa1);
                read_sb(psb);
                afc = read_a(std::integral_constant<int, 0>{}, pa0, pa1);
                sac = read_sa(std::integral_constant<int, 0>{}, psa);
            }
        };

        // stage 0 (step 0) has landed: step 1 goes out, step 0's operands are
        // read.  The previous tile's stores, issued after step 0's DMA, may
        // stay in flight (a wave that issues no DMA has only those).
        if (stores_out) wait_vmcnt<NST>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (nkb > 1) issue(sbase + SM::STAGE, 1, cs);
        read_step(sbase);
        for (int kb0 = 0; kb0 < nkb; kb0 += 2) {
            kstep(std::integral_constant<int, 0>{}, kb0);
            if (kb0 + 1 < nkb) kstep(std::integral_constant<int, 1>{}, kb0 + 1);
        }
        // the next tile's first step goes out now and overlaps the epilogue
        uint16_t* dst = dst_of(cp);
        step_pos(cp);
        have = cp.j < Lne;
        if (have) {
            cs = src_of(cp);
            issue(sbase, 0, cs);
        }
        // bf16 from the accumulators; two cross-lane swaps per pair of
        // n-subtiles give each lane 8 consecutive columns (one 16-byte store),
        // then the lanes of rows 2u and 2u + 1 trade halves so that each store
        // writes whole 128-byte lines, as in wgrad_fp8_kernel's epilogue
        uint8_t* d = reinterpret_cast<uint8_t*>(dst);
        uint32_t o_lane = o_lane0;  // 32-bit lane offset; the row block is a uniform base
        pin(o_lane);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            uint8_t* drow = d + (int64_t)mi * 16 * N * 2;
            uint32_t x[NI], y[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const v4f a = acc[mi][ni];
                x[ni] = cvt_bf16x2(a.x, a.y);
                y[ni] = cvt_bf16x2(a.z, a.w);
            }
#pragma unroll
            for (int ni = 0; ni < NI; ni += 2) {
                swap32(x[ni], x[ni + 1]);
                swap32(y[ni], y[ni + 1]);
                swap16(x[ni], x[ni + 1]);
                swap16(y[ni], y[ni + 1]);
            }
            const u32x4 p0 = {x[0], y[0], x[1], y[1]}, p1 = {x[2], y[2], x[3], y[3]};
            const u32x4 snd = odd_row ? p0 : p1;
            u32x4 r;
#pragma unroll
            for (int c = 0; c < 4; ++c) r[c] = (uint32_t)__builtin_amdgcn_mov_dpp((int)snd[c], 0xB1, 0xF, 0xF, false);
            st_stream(reinterpret_cast<u32x4*>(drow + o_lane), odd_row ? r : p0);
            st_stream(reinterpret_cast<u32x4*>(drow + o_lane + 2 * N), odd_row ? p1 : r);
        }
        stores_out = true;
    }

    zero_fill_empty(g, tid);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_grouped_gemm_fp8_wgrad(const uint8_t* aT, const float* aT_s, const uint8_t* bT,
                                          const float* bT_s, const int32_t* offsets, int32_t L, int64_t row_cap,
                                          int32_t M, int32_t N, uint16_t* dW, int32_t flags, hipStream_t stream) {
    MOE_REQUIRE((flags & ~(MOE_SCALE_POW2 | MOE_GEMM_TILE128)) == 0, MOE_ERR_UNSUPPORTED,
                "grouped_gemm_wgrad: unknown flags 0x%x", flags);
    const bool p2 = (flags & MOE_SCALE_POW2) != 0;
    MOE_REQUIRE(L >= 1 && L <= WMAXL, MOE_ERR_SHAPE, "grouped_gemm_wgrad: L=%d outside [1, %d]", L, WMAXL);
    // segment starts are kept as 32-bit values on the device
    MOE_REQUIRE(row_cap >= 0 && row_cap % WBK == 0 && row_cap < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: row_cap=%lld must be a multiple of 128 below 2^31", (long long)row_cap);
    MOE_REQUIRE(M > 0 && M % WBM == 0 && N > 0 && N % 128 == 0, MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: M=%d and N=%d must be multiples of 128", M, N);
    MOE_REQUIRE((int64_t)L * (M / WBM) * (N / 128) < ((int64_t)1 << 31), MOE_ERR_SHAPE,
                "grouped_gemm_wgrad: too many tiles");
    MOE_REQUIRE(aT && aT_s && bT && bT_s && offsets && dW, MOE_ERR_NULL, "grouped_gemm_wgrad: NULL argument");
    const bool wide = p2 && M % 256 == 0 && N % 256 == 0 && !(flags & MOE_GEMM_TILE128);
    const int BMt = wide ? 256 : WBM, BNt = (wide || N % 256 == 0) ? 256 : 128;
    const int nfast = N < M ? 1 : 0;
    // The fast index runs in groups of 8 tiles when its count allows: the 32
    // tiles an XCD runs side by side then cover 8 x 4 tiles, so they read 8
    // tiles of one operand and 4 of the other instead of all of one.
    const int ft = nfast ? N / BNt : M / BMt;
    const int gf = (ft > 8 && ft % 8 == 0) ? 8 : ft;
    WgradArgs a{aT, aT_s, bT, bT_s, offsets, L, row_cap, M, N, nfast, gf, dW, 1, 0x7FFFFFFF, 1};
    const int grid = (num_cus() + 7) / 8 * 8;  // persistent, one block per CU
    auto go = [&](auto kern, const WgradArgs& args) { kern<<<dim3(grid), dim3(WTHREADS), 0, stream>>>(args); };
    if (wide) {
        go(wgrad_wide_kernel, a);
    } else if (N % 256 == 0 && !(flags & MOE_GEMM_TILE128)) {
        // experts of at most ARES_KB token blocks keep their A operand in LDS;
        // any longer ones (only possible when row_cap allows) stream both
        WgradArgs ar = a;
        ar.kb_max = ARES_KB;
        p2 ? go(wgrad_ares_kernel<true>, ar) : go(wgrad_ares_kernel<false>, ar);
        MOE_LAUNCH_CHECK("wgrad_ares_kernel");
        if (row_cap / WBK > ARES_KB) {
            WgradArgs as = a;
            as.kb_min = ARES_KB + 1;
            as.zfill = 0;
            p2 ? go(wgrad_fp8_kernel<256, true>, as) : go(wgrad_fp8_kernel<256, false>, as);
        }
    } else if (N % 256 == 0) {
        p2 ? go(wgrad_fp8_kernel<256, true>, a) : go(wgrad_fp8_kernel<256, false>, a);
    } else {
        p2 ? go(wgrad_fp8_kernel<128, true>, a) : go(wgrad_fp8_kernel<128, false>, a);
    }
    MOE_LAUNCH_CHECK("wgrad_fp8_kernel");
    return MOE_OK;
}
