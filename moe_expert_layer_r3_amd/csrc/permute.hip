// Dispatch on one GPU's share of experts ("RL at 1T scale", sections "Wide
// Expert Parallelism" and "Expert Parallel"): the per-layer dispatch becomes a
// local, stable, expert-grouped permutation of the (token, slot) pairs.
//
//   1. hist    : per chunk of PCHUNK pairs, count local pairs per expert (LDS)
//   2. scan    : per expert, exclusive scan of the chunk counts (one wave per
//                expert, shuffle prefix over 64 chunks at a time); counts; the
//                128-aligned offsets; padding rows of row_pair = -1
//   3. scatter : per chunk, rank every pair among the earlier pairs of its
//                expert (wave ballots, in pair order) and write row_pair /
//                pair_row -- deterministic, no order-dependent atomics; the
//                per-expert row bases of the chunk are staged in LDS first.
//                When the chunk counts are few (nchunk * L <= SCAN_FOLD), step
//                2 runs inside this kernel instead: every block reads all
//                chunk counts and forms its own bases and the offsets.
//   4. gather  : one workgroup per token: its local rows are read once as
//                uniform values, the row of x is read once, quantised to
//                1x128 e4m3 once, and written to each of its local rows.
// Chunks are small (1024 pairs) so that even a few thousand tokens spread the
// index work over many workgroups; every step is latency-bound, not
// bandwidth-bound.
#include <mutex>

#include "common.hpp"

namespace moe {

constexpr int PCHUNK = 1024;       // pairs per chunk (one block)
constexpr int PBLOCK = 256;        // threads per block in hist / scatter
constexpr int PWAVES = PBLOCK / 64;
constexpr int PER_WAVE = PCHUNK / PWAVES;  // 256 consecutive pairs per wave
constexpr int MAXL = 1024;

constexpr int SCAN_FOLD = 16384;   // chunk counts (int32) a scatter block reads to fold the scan in

// Lanes of the wave whose local expert id equals this lane's (le >= 0): one
// ballot per bit of the id (nb = bits of L - 1) instead of one per distinct id.
// Lanes with le < 0 are in no mask.
__device__ __forceinline__ uint64_t same_expert(int le, int nb) {
    uint64_t m = __ballot(le >= 0);
    for (int b = 0; b < nb; ++b) {
        const bool bit = (le >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}
__device__ __forceinline__ int expert_bits(int L) { return L > 1 ? 32 - __clz(L - 1) : 0; }

__global__ __launch_bounds__(PBLOCK) void perm_hist_kernel(const int32_t* __restrict__ ids, int64_t P, int e0,
                                                           int L, int32_t* __restrict__ chunk_counts) {
    __shared__ int cnt[MAXL];
    for (int e = threadIdx.x; e < L; e += PBLOCK) cnt[e] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nb = expert_bits(L);
    const int64_t base = (int64_t)blockIdx.x * PCHUNK;
    // all of the thread's ids are requested before any is used (a pair past P
    // reads the last pair's id and is dropped)
    constexpr int IT = PCHUNK / PBLOCK;
    int les[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = base + it * PBLOCK + threadIdx.x;
        les[it] = ids[p < P ? p : P - 1];
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int64_t p = base + it * PBLOCK + threadIdx.x;
        int le = les[it] - e0;
        if (p >= P || le < 0 || le >= L) le = -1;
        // the first lane of each expert adds the wave's count (distinct addresses)
        const uint64_t m = same_expert(le, nb);
        if (le >= 0 && (m & lt_mask) == 0) atomicAdd(&cnt[le], (int)__popcll(m));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < L; e += PBLOCK) chunk_counts[(int64_t)blockIdx.x * L + e] = cnt[e];
}

// Single block of 1024 threads (16 waves).  Wave w handles experts w, w + 16,
// ... for the chunk prefixes and the padding rows; thread e owns expert e for
// the scan over experts (wave shuffles, one LDS round for the wave totals).
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunk, int L,
                                                         int64_t row_cap, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_pair,
                                                         int32_t* __restrict__ status) {
    __shared__ int tot[MAXL];
    __shared__ int64_t wsum[16];
    __shared__ int64_t ends[MAXL];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // exclusive prefix of each expert's chunk counts, in place
    for (int e = wave; e < L; e += 16) {
        int carry = 0;
        for (int c0 = 0; c0 < nchunk; c0 += 64) {
            const int c = c0 + lane;
            const int v = c < nchunk ? chunk_counts[(int64_t)c * L + e] : 0;
            int x = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            if (c < nchunk) chunk_counts[(int64_t)c * L + e] = carry + x - v;
            carry += __builtin_amdgcn_readlane(x, 63);
        }
        if (lane == 0) tot[e] = carry;
    }
    __syncthreads();
    // inclusive scan of the 128-aligned segment sizes over experts
    const int e = threadIdx.x;
    const int run = e < L ? tot[e] : 0;
    const int64_t padded = ((int64_t)run + MOE_ROW_ALIGN - 1) / MOE_ROW_ALIGN * MOE_ROW_ALIGN;
    int64_t x = padded;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    for (int w = 0; w < wave; ++w) x += wsum[w];
    if (e < L) {
        ends[e] = x;
        counts[e] = run;
        offsets[e + 1] = (int32_t)(x > 0x7FFFFFFF ? 0x7FFFFFFF : x);
        if (e == 0) offsets[0] = 0;
        if (e == L - 1 && x > row_cap && status) atomicOr(status, MOE_FLAG_ROW_CAP);
    }
    __syncthreads();
    // padding rows of each segment (fewer than 128): row_pair = -1
    for (int e2 = wave; e2 < L; e2 += 16) {
        const int64_t end = ends[e2];
        const int c = tot[e2];
        const int64_t start = end - ((int64_t)c + MOE_ROW_ALIGN - 1) / MOE_ROW_ALIGN * MOE_ROW_ALIGN;
        for (int64_t r = start + c + lane; r < end; r += 64)
            if (r < row_cap) row_pair[r] = -1;
    }
}

// FOLD: chunk_counts holds the raw counts of every chunk (nchunk * L <=
// SCAN_FOLD); each block forms its chunk's bases and the 128-aligned offsets
// itself, and block 0 writes counts, offsets, the padding rows and the row-cap
// flag (what perm_scan_kernel does otherwise).  Without FOLD, chunk_counts
// holds the scan's exclusive chunk prefixes.
template <bool FOLD>
__global__ __launch_bounds__(PBLOCK) void perm_scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int e0,
                                                              int L, int64_t row_cap, int nchunk,
                                                              const int32_t* __restrict__ chunk_counts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_pair,
                                                              int32_t* __restrict__ pair_row,
                                                              int32_t* __restrict__ status) {
    // run[w][e]: pairs of expert e seen so far by wave w (first pass: totals);
    // base[e]: first row of this chunk's pairs of expert e
    __shared__ int run[PWAVES][MAXL];
    __shared__ int64_t base[MAXL];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t wbase = (int64_t)blockIdx.x * PCHUNK + (int64_t)wave * PER_WAVE;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nb = expert_bits(L);

    // the wave's local expert ids, loaded once for both passes: every load is
    // issued before any is used and before the bases are formed (a pair past
    // P reads the last pair's id and is dropped)
    int les[PER_WAVE / 64];
#pragma unroll
    for (int it = 0; it < PER_WAVE / 64; ++it) {
        const int64_t p = wbase + it * 64 + lane;
        les[it] = ids[p < P ? p : P - 1];
    }
#pragma unroll
    for (int it = 0; it < PER_WAVE / 64; ++it) {
        const int64_t p = wbase + it * 64 + lane;
        int le = les[it] - e0;
        if (p >= P || le < 0 || le >= L) le = -1;
        les[it] = le;
    }
    for (int e = threadIdx.x; e < L; e += PBLOCK)
        for (int w = 0; w < PWAVES; ++w) run[w][e] = 0;
    if constexpr (FOLD) {
        // per expert: its pairs in the chunks before this one (pre) and in all
        // chunks (tot); thread (cs, e) sums chunks cs, cs + cstep, ...
        __shared__ int pre[MAXL], tot[MAXL];
        __shared__ int64_t wsum[PWAVES];
        for (int e = threadIdx.x; e < L; e += PBLOCK) {
            pre[e] = 0;
            tot[e] = 0;
        }
        __syncthreads();
        const int cstep = L <= PBLOCK ? PBLOCK / L : 1;
        for (int e0t = 0; e0t < L; e0t += PBLOCK) {
            const int e = e0t + (L <= PBLOCK ? (int)threadIdx.x % L : (int)threadIdx.x);
            const int cs = L <= PBLOCK ? (int)threadIdx.x / L : 0;
            if (e < L && cs < cstep) {
                // 16 chunk counts requested at a time (indices past the last
                // chunk read the last one and are not added)
                constexpr int CB = 16;
                int a = 0, t = 0;
                for (int c0 = cs; c0 < nchunk; c0 += CB * cstep) {
                    int v[CB];
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        const int c = c0 + j * cstep;
                        v[j] = chunk_counts[(int64_t)(c < nchunk ? c : nchunk - 1) * L + e];
                    }
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        const int c = c0 + j * cstep;
                        const int w = c < nchunk ? v[j] : 0;
                        t += w;
                        a += c < (int)blockIdx.x ? w : 0;
                    }
                }
                atomicAdd(&pre[e], a);
                atomicAdd(&tot[e], t);
            }
        }
        __syncthreads();
        // inclusive scan over experts of the 128-aligned segment sizes: each
        // thread sums its run of consecutive experts, then a block scan
        const int per = (L + PBLOCK - 1) / PBLOCK;
        const int ea = threadIdx.x * per, eb = min(L, ea + per);
        int64_t own = 0;
        for (int e = ea; e < eb; ++e)
            own += ((int64_t)tot[e] + MOE_ROW_ALIGN - 1) / MOE_ROW_ALIGN * MOE_ROW_ALIGN;
        int64_t x = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        for (int w = 0; w < wave; ++w) x += wsum[w];
        int64_t start = x - own;  // first row of expert ea
        for (int e = ea; e < eb; ++e) {
            const int c = tot[e];
            const int64_t end = start + ((int64_t)c + MOE_ROW_ALIGN - 1) / MOE_ROW_ALIGN * MOE_ROW_ALIGN;
            base[e] = start + pre[e];
            if (blockIdx.x == 0) {
                counts[e] = c;
                offsets[e + 1] = (int32_t)(end > 0x7FFFFFFF ? 0x7FFFFFFF : end);
                if (e == 0) offsets[0] = 0;
                if (e == L - 1 && end > row_cap && status) atomicOr(status, MOE_FLAG_ROW_CAP);
                for (int64_t r = start + c; r < end && r < row_cap; ++r) row_pair[r] = -1;  // < 128 rows
            }
            start = end;
        }
    } else {
        for (int e = threadIdx.x; e < L; e += PBLOCK)
            base[e] = (int64_t)offsets[e] + chunk_counts[(int64_t)blockIdx.x * L + e];
    }
    __syncthreads();

    // pass 1: per-wave totals per expert; the first lane of each expert adds
    // the count (distinct addresses within an instruction)
    uint64_t mk[PER_WAVE / 64];
#pragma unroll
    for (int it = 0; it < PER_WAVE / 64; ++it) {
        const int le = les[it];
        mk[it] = same_expert(le, nb);
        if (le >= 0 && (mk[it] & lt_mask) == 0) run[wave][le] += (int)__popcll(mk[it]);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // exclusive prefix over waves, per expert
    for (int e = threadIdx.x; e < L; e += PBLOCK) {
        int acc = 0;
        for (int w = 0; w < PWAVES; ++w) {
            int v = run[w][e];
            run[w][e] = acc;
            acc += v;
        }
    }
    __syncthreads();
    // pass 2: ranks in pair order (earlier waves, earlier iterations, earlier
    // lanes), write rows
#pragma unroll
    for (int it = 0; it < PER_WAVE / 64; ++it) {
        const int64_t p = wbase + it * 64 + lane;
        const int le = les[it];
        const uint64_t m = mk[it];
        int64_t row = -1;
        int before = 0;
        if (le >= 0) {
            before = run[wave][le];
            row = base[le] + before + __popcll(m & lt_mask);
        }
        __builtin_amdgcn_wave_barrier();
        if (le >= 0 && (m & lt_mask) == 0) run[wave][le] = before + (int)__popcll(m);
        __builtin_amdgcn_wave_barrier();
        if (p < P) {
            if (row >= row_cap) row = -1;
            pair_row[p] = (int32_t)row;
            if (row >= 0) row_pair[row] = (int32_t)p;
        }
    }
}

// Token-major gather with fused 1x128 quantisation: one workgroup per token.
// The token's k local rows are uniform (scalar loads, k <= 16); each 16-lane
// group covers one 128-column tile with 8 bf16 per lane, so the tile's amax is
// a 16-lane reduction.  The row's loads are issued together (up to GQ_LOADS
// passes of 256 lanes x 8 columns) before any store.
constexpr int GQ_THREADS = 256;
constexpr int GQ_LOADS = 4;

template <bool P2>
__global__ __launch_bounds__(GQ_THREADS) void gather_quant_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                                  int d, int k,
                                                                  const int32_t* __restrict__ pair_row,
                                                                  uint16_t* __restrict__ x_perm,
                                                                  uint8_t* __restrict__ xq,
                                                                  float* __restrict__ xq_s, int64_t row_cap) {
    const int64_t t = blockIdx.x;
    const uint16_t* xr = x + t * d;
    // the routing slots first: a token without a local row reads nothing of x
    // (issuing part of the row together with the slots, to save a latency for
    // tokens with local rows, measured slower at the ep8 shape, where a third
    // of the tokens have none: 22 MB more read, 51 vs 49 us)
    int r[16];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        r[j] = j < k ? pair_row[t * k + j] : -1;
        any |= r[j] >= 0;
    }
    if (!any) return;
    uint4 raw[GQ_LOADS];
#pragma unroll
    for (int i = 0; i < GQ_LOADS; ++i) {
        const int col = (i * GQ_THREADS + threadIdx.x) * 8;
        if (col < d) raw[i] = *reinterpret_cast<const uint4*>(xr + col);
    }
    const int sub = threadIdx.x & 15;
    for (int c0 = 0; c0 < d; c0 += GQ_LOADS * GQ_THREADS * 8) {
        if (c0 > 0) {
#pragma unroll
            for (int i = 0; i < GQ_LOADS; ++i) {
                const int col = c0 + (i * GQ_THREADS + threadIdx.x) * 8;
                if (col < d) raw[i] = *reinterpret_cast<const uint4*>(xr + col);
            }
        }
#pragma unroll
        for (int i = 0; i < GQ_LOADS; ++i) {
            const int col = c0 + (i * GQ_THREADS + threadIdx.x) * 8;
            // d % 128 == 0: a 16-lane group is entirely in or out of range
            if (col >= d) continue;
            const int tile = col >> 7;
            uint2 packed = make_uint2(0, 0);
            float s = 0.f;
            if (xq) {
                float v[8];
                v[0] = bf16_lo(raw[i].x); v[1] = bf16_hi(raw[i].x);
                v[2] = bf16_lo(raw[i].y); v[3] = bf16_hi(raw[i].y);
                v[4] = bf16_lo(raw[i].z); v[5] = bf16_hi(raw[i].z);
                v[6] = bf16_lo(raw[i].w); v[7] = bf16_hi(raw[i].w);
                float am = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) am = fmaxf(am, fabsf(v[q]));
                am = group_max<16>(am);
                const TileScale ts = tile_scale_t<P2>(am);
                s = ts.s;
                packed.x = cvt_e4m3x4(v[0] * ts.inv, v[1] * ts.inv, v[2] * ts.inv, v[3] * ts.inv);
                packed.y = cvt_e4m3x4(v[4] * ts.inv, v[5] * ts.inv, v[6] * ts.inv, v[7] * ts.inv);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j >= k || r[j] < 0) continue;
                const int64_t row = r[j];
                if (x_perm) *reinterpret_cast<uint4*>(x_perm + row * d + col) = raw[i];
                if (xq) {
                    *reinterpret_cast<uint2*>(xq + row * d + col) = packed;
                    if (sub == 0) xq_s[tile * row_cap + row] = s;  // K-block-major scales
                }
            }
        }
    }
}

}  // namespace moe

using namespace moe;

static int64_t perm_chunks(int64_t T, int32_t k) { return (T * k + PCHUNK - 1) / PCHUNK; }

extern "C" int moe_permute_workspace(int64_t T, int32_t k, int32_t L, size_t* bytes) {
    MOE_REQUIRE(bytes, MOE_ERR_NULL, "permute_workspace: NULL bytes");
    MOE_REQUIRE(T >= 0 && k >= 1 && k <= 16 && L >= 1 && L <= MAXL, MOE_ERR_SHAPE,
                "permute_workspace: bad T/k/L");
    int64_t n = perm_chunks(T, k);
    *bytes = (size_t)((n > 0 ? n : 1) * L * sizeof(int32_t));
    return MOE_OK;
}

// Validation and launches shared by moe_permute and moe_permute_noalloc; the
// chunk counts live in `chunk` (nchunk * L int32), written in full by the hist
// kernel before the scan and the scatter read them.
static int permute_check(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L, int64_t row_cap,
                         int32_t* counts, int32_t* offsets, int32_t* row_pair, int32_t* pair_row,
                         const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq, float* xq_s,
                         int32_t quant_flags) {
    MOE_REQUIRE(T >= 0 && T <= ((int64_t)1 << 31) / 16, MOE_ERR_SHAPE, "permute: bad T=%lld", (long long)T);
    MOE_REQUIRE(k >= 1 && k <= 16, MOE_ERR_SHAPE, "permute: k=%d outside [1, 16]", k);
    MOE_REQUIRE(L >= 1 && L <= MAXL && e0 >= 0, MOE_ERR_SHAPE, "permute: L=%d outside [1, 1024] or e0<0", L);
    MOE_REQUIRE(row_cap >= 0 && row_cap % MOE_ROW_ALIGN == 0 && row_cap <= 0x7FFFFFFF, MOE_ERR_SHAPE,
                "permute: row_cap=%lld must be a multiple of 128 below 2^31", (long long)row_cap);
    MOE_REQUIRE(counts && offsets && (T == 0 || (ids && pair_row)) && (row_cap == 0 || row_pair), MOE_ERR_NULL,
                "permute: NULL ids/counts/offsets/row_pair/pair_row");
    MOE_REQUIRE(quant_flags == 0 || quant_flags == MOE_SCALE_POW2, MOE_ERR_UNSUPPORTED,
                "permute: unknown quant_flags 0x%x", quant_flags);
    if (x) {
        MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "permute: d=%d must be a positive multiple of 128", d);
        MOE_REQUIRE(x_perm || xq, MOE_ERR_NULL, "permute: x given but neither x_perm nor xq");
        MOE_REQUIRE(!xq || xq_s, MOE_ERR_NULL, "permute: xq without xq_s");
    } else {
        MOE_REQUIRE(!x_perm && !xq, MOE_ERR_NULL, "permute: x_perm/xq given without x");
    }
    return MOE_OK;
}

static int permute_launch(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L, int64_t row_cap,
                          int32_t* counts, int32_t* offsets, int32_t* row_pair, int32_t* pair_row,
                          const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq, float* xq_s,
                          int32_t quant_flags, int32_t* chunk, int32_t* dev_status, hipStream_t stream) {
    const int64_t P = T * k;
    const int nchunk = (int)perm_chunks(T, k);
    if (nchunk > 0) {
        perm_hist_kernel<<<dim3(nchunk), dim3(PBLOCK), 0, stream>>>(ids, P, e0, L, chunk);
        MOE_LAUNCH_CHECK("perm_hist_kernel");
    }
    if (nchunk > 0 && (int64_t)nchunk * L <= SCAN_FOLD) {
        perm_scatter_kernel<true><<<dim3(nchunk), dim3(PBLOCK), 0, stream>>>(
            ids, P, e0, L, row_cap, nchunk, chunk, counts, offsets, row_pair, pair_row, dev_status);
        MOE_LAUNCH_CHECK("perm_scatter_kernel");
    } else {
        perm_scan_kernel<<<dim3(1), dim3(1024), 0, stream>>>(chunk, nchunk, L, row_cap, counts, offsets, row_pair,
                                                             dev_status);
        MOE_LAUNCH_CHECK("perm_scan_kernel");
        if (nchunk > 0) {
            perm_scatter_kernel<false><<<dim3(nchunk), dim3(PBLOCK), 0, stream>>>(
                ids, P, e0, L, row_cap, nchunk, chunk, counts, offsets, row_pair, pair_row, dev_status);
            MOE_LAUNCH_CHECK("perm_scatter_kernel");
        }
    }
    if (x && T > 0) {
        auto go = [&](auto kern) {
            kern<<<dim3((unsigned)T), dim3(GQ_THREADS), 0, stream>>>(x, T, d, k, pair_row, x_perm, xq, xq_s, row_cap);
        };
        quant_flags ? go(gather_quant_kernel<true>) : go(gather_quant_kernel<false>);
        MOE_LAUNCH_CHECK("gather_quant_kernel");
    }
    return MOE_OK;
}

extern "C" int moe_permute(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L, int64_t row_cap,
                           int32_t* counts, int32_t* offsets, int32_t* row_pair, int32_t* pair_row,
                           const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq, float* xq_s,
                           int32_t quant_flags, void* ws, size_t ws_bytes, int32_t* dev_status,
                           hipStream_t stream) {
    int rc = permute_check(ids, T, k, e0, L, row_cap, counts, offsets, row_pair, pair_row, x, d, x_perm, xq, xq_s,
                           quant_flags);
    if (rc != MOE_OK) return rc;
    size_t need = 0;
    moe_permute_workspace(T, k, L, &need);
    MOE_REQUIRE(ws && ws_bytes >= need, MOE_ERR_WORKSPACE, "permute: workspace %zu < %zu bytes", ws_bytes, need);
    return permute_launch(ids, T, k, e0, L, row_cap, counts, offsets, row_pair, pair_row, x, d, x_perm, xq, xq_s,
                          quant_flags, static_cast<int32_t*>(ws), dev_status, stream);
}

// ---------------------------------------------------------------- allocation-free variant
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the chunk counts live in this file-scope
// device array instead of a caller workspace.  Each GPU holds its own copy
// until the process ends; every call on a GPU shares it, so calls that overlap
// on one GPU (concurrent streams) race.  Nothing in it needs clearing: the
// hist kernel writes every count the scan and scatter read.
namespace moe {
constexpr size_t PERMUTE_SCRATCH_BYTES = MOE_PERMUTE_NOALLOC_MAX_WS;
static __device__ __align__(256) int32_t scratch[PERMUTE_SCRATCH_BYTES / sizeof(int32_t)];

// Device address of `scratch` on the current device, looked up once per device
// (the array's name in host code is only a stand-in for the symbol).
static int scratch_address(int32_t** out) {
    constexpr int MAXDEV = 64;
    static int32_t* ptrs[MAXDEV] = {};
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    MOE_REQUIRE(e == hipSuccess, MOE_ERR_HIP, "permute_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    MOE_REQUIRE(dev >= 0 && dev < MAXDEV, MOE_ERR_UNSUPPORTED, "permute_noalloc: device %d >= %d", dev, MAXDEV);
    std::lock_guard<std::mutex> lk(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        MOE_REQUIRE(e == hipSuccess && p, MOE_ERR_HIP, "permute_noalloc: hipGetSymbolAddress: %s",
                    hipGetErrorString(e));
        ptrs[dev] = static_cast<int32_t*>(p);
    }
    *out = ptrs[dev];
    return MOE_OK;
}
}  // namespace moe

extern "C" int moe_permute_noalloc(const int32_t* ids, int64_t T, int32_t k, int32_t e0, int32_t L,
                                   int64_t row_cap, int32_t* counts, int32_t* offsets, int32_t* row_pair,
                                   int32_t* pair_row, const uint16_t* x, int32_t d, uint16_t* x_perm, uint8_t* xq,
                                   float* xq_s, int32_t quant_flags, int32_t* dev_status, hipStream_t stream) {
    int rc = permute_check(ids, T, k, e0, L, row_cap, counts, offsets, row_pair, pair_row, x, d, x_perm, xq, xq_s,
                           quant_flags);
    if (rc != MOE_OK) return rc;
    size_t need = 0;
    moe_permute_workspace(T, k, L, &need);
    MOE_REQUIRE(need <= PERMUTE_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
                "permute_noalloc: T=%lld, k=%d, L=%d need %zu bytes of chunk counts, more than the %zu bytes of "
                "its device scratch (use moe_permute with a workspace)",
                (long long)T, k, L, need, PERMUTE_SCRATCH_BYTES);
    int32_t* chunk = nullptr;
    rc = scratch_address(&chunk);
    if (rc != MOE_OK) return rc;
    return permute_launch(ids, T, k, e0, L, row_cap, counts, offsets, row_pair, pair_row, x, d, x_perm, xq, xq_s,
                          quant_flags, chunk, dev_status, stream);
}
