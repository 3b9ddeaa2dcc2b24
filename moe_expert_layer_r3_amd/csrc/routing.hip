// Routing kernels: wavefront top-k with softmax gates (optionally recording the
// selection for Router Replay), the Router Replay load, and the gate backward.
//
// Router Replay follows "RL at 1T scale", section "Router Replay": the recorded
// payload [num_layers, top_k, seq_len] stays on the device and is consumed by
// device kernels only.
#include "common.hpp"
#include "gate_parts.hpp"

namespace moe {

constexpr int MAXK = 16;

// Selection key of (logit x, expert e): one 64-bit integer whose order is the
// routing order (value descending, then id ascending), so a pick is a plain
// unsigned max and every key of a row is distinct.
//   high word: the float's bits mapped monotonically to unsigned (negative
//              values bit-inverted, positive ones with the sign bit set); x is
//              canonicalised by adding +0 first, so -0 and +0 share a key and
//              fall back to the id order, as IEEE comparison has them equal;
//              NaN takes 1, below every number (NaN sorts last)
//   low word : ~e, larger for the lower id
// Key 0 means "no candidate" (a lane slot past E).  Because the picks come out
// in strictly descending key order, the values still available in a round are
// exactly those below the previous pick: no per-value taken flags.
__device__ __forceinline__ uint64_t route_key(float x, int e) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    if (x != x) hi = 1u;
    return ((uint64_t)hi << 32) | (uint32_t)~e;
}
__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t hi = (uint32_t)(key >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}
__device__ __forceinline__ int route_key_id(uint64_t key) { return (int)~(uint32_t)key; }

// A key moved across the 16-lane row by a DPP pattern (no LDS trip).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One wavefront per token row.  Lane l holds logits l, l+64, ... (VPL values);
// k rounds of a wave-wide arg-max over route_key pick the slots in order.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                   int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ rec, int64_t rec_stride, int64_t s0) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= T) return;
    const float* src = logits + row * E;
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? route_key(src[e], e) : 0ull;
    }
    uint64_t thr = ~0ull, mine = 0ull;
    for (int s = 0; s < k; ++s) {
        uint64_t b = 0ull;
#pragma unroll
        for (int i = 0; i < VPL; ++i) b = (key[i] < thr && key[i] > b) ? key[i] : b;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const uint64_t o = __shfl_xor(b, m);
            b = o > b ? o : b;
        }
        thr = b;
        if (lane == s) mine = b;
    }
    const float my_val = route_key_value(mine);
    const int my_id = route_key_id(mine);
    // softmax over the selection; slot 0 holds the max
    float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
    float ex = lane < k ? expf(my_val - m) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; ++j)  // ascending slot order; j is uniform: a register read, no LDS trip
        sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    if (lane < k) {
        ids[row * k + lane] = my_id;
        w[row * k + lane] = ex / sum;
        if (rec) rec[(int64_t)lane * rec_stride + s0 + row] = my_id;
    }
}

// Keys sorted descending in place: Batcher's odd-even merge sort, a fixed
// network of compare-exchanges (63 for N = 16) that unrolls to straight-line
// code with independent exchanges at each level.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1) {
#pragma unroll
        for (int q = p; q >= 1; q >>= 1) {
#pragma unroll
            for (int j = q % p; j <= N - 1 - q; j += 2 * q) {
#pragma unroll
                for (int i = 0; i <= (q - 1 < N - j - q - 1 ? q - 1 : N - j - q - 1); ++i) {
                    if ((i + j) / (2 * p) == (i + j + q) / (2 * p)) {
                        const uint64_t a = key[i + j], b = key[i + j + q];
                        const bool sw = b > a;
                        key[i + j] = sw ? b : a;
                        key[i + j + q] = sw ? a : b;
                    }
                }
            }
        }
    }
}

// Sixteen lanes per token row, for E <= 16 * VPL <= 256: lane l of a group
// holds logits VPL*l .. VPL*l + VPL - 1 (a contiguous run) and sorts their
// route_keys descending.  Pick s is then the 16-lane max of the lanes' first
// keys (four DPP steps), and the lane that held it moves its next key up: the
// picks are the row's keys in descending order, one max chain of four steps
// per pick instead of a scan of VPL keys.  A lane gives up at most k keys, so
// KT >= min(k, VPL) of its sorted keys are kept.
template <int VPL, int KT>
__global__ __launch_bounds__(256) void topk16_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                     int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                                     int32_t* __restrict__ rec, int64_t rec_stride, int64_t s0) {
    const int lane = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4);
    // every lane takes part in the shuffles; rows past T compute on row 0 and store nothing
    const bool live = row < T;
    const float* src = logits + (live ? row : 0) * E;
    float v[VPL];
    if (VPL % 4 == 0 && E % 4 == 0 && lane * VPL + VPL <= E) {
        // the lane's whole run is in the row and 16-byte aligned
#pragma unroll
        for (int c = 0; c < VPL / 4; ++c) {
            const float4 q = reinterpret_cast<const float4*>(src + lane * VPL)[c];
            v[4 * c] = q.x;
            v[4 * c + 1] = q.y;
            v[4 * c + 2] = q.z;
            v[4 * c + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane * VPL + i;
            v[i] = e < E ? src[e] : -INFINITY;
        }
    }
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane * VPL + i;
        key[i] = e < E ? route_key(v[i], e) : 0ull;
    }
    sort_desc<VPL>(key);
    uint64_t h[KT];
#pragma unroll
    for (int i = 0; i < KT; ++i) h[i] = key[i];
    uint64_t mine = 0ull;
    for (int s = 0; s < k; ++s) {
        // max over the 16-lane group: swap neighbours, swap pairs (each lane
        // then holds its quad's max), mirror within 8 lanes, mirror within 16
        uint64_t b = h[0];
        b = umax64(b, dpp_key<0xB1>(b));
        b = umax64(b, dpp_key<0x4E>(b));
        b = umax64(b, dpp_key<0x141>(b));
        b = umax64(b, dpp_key<0x140>(b));
        // keys are distinct, so exactly one lane held b (a lane whose keys
        // ran out holds 0, and with k <= E no pick is 0).  The move is a bit
        // blend under an all-ones mask that the optimiser cannot see through
        // (as selects on the flag it becomes per-lane index arithmetic with
        // select chains over all KT keys)
        uint32_t m32 = h[0] == b ? ~0u : 0u;
        asm volatile("" : "+v"(m32));
        const uint64_t m = ((uint64_t)m32 << 32) | m32;
#pragma unroll
        for (int i = 0; i + 1 < KT; ++i) h[i] = (h[i + 1] & m) | (h[i] & ~m);
        h[KT - 1] &= ~m;
        if (lane == s) mine = b;
    }
    const float my_val = route_key_value(mine);
    const int my_id = route_key_id(mine);
    // softmax over the selection; slot 0 holds the max
    const float m = __shfl(my_val, 0, 16);
    const float ex = lane < k ? expf(my_val - m) : 0.f;
    float sum = 0.f;
    // ascending slot order; all shuffles issued before the first add
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
        const float o = __shfl(ex, j, 16);
        if (j < k) sum += o;
    }
    if (live && lane < k) {
        ids[row * k + lane] = my_id;
        w[row * k + lane] = ex / sum;
        if (rec) rec[(int64_t)lane * rec_stride + s0 + row] = my_id;
    }
}

// The same routing order as a double.  For ord = the high word of route_key
// (the float's order-preserving bits, NaN -> 1) the 64-bit pattern
// 2^62 + ord * 2^30 + (1023 - e) is a positive, normal, finite IEEE double
// (its exponent field is 0x400 + the top ten bits of ord, at most 0x7FE
// because no non-NaN float maps above 0xFF800000), and such doubles order as
// their bit patterns do: by ord, then by the lower id.  A compare-exchange is
// then one v_max_f64 and one v_min_f64, with no lane mask and no select.
// 0.0 marks "no candidate" and sits below every key.  Needs e < 1024.
__device__ __forceinline__ double route_dkey(float x, int e) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    uint32_t ord = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    ord = x != x ? 1u : ord;
    const uint32_t hi = __builtin_amdgcn_alignbit(1u, ord, 2);  // 0x40000000 | ord >> 2
    const uint32_t lo = (ord << 30) | (uint32_t)(1023 - e);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t route_dkey_ord(double d) {
    const uint64_t b = __builtin_bit_cast(uint64_t, d);
    return ((uint32_t)(b >> 32) << 2) | ((uint32_t)b >> 30);
}
__device__ __forceinline__ int route_dkey_id(double d) {
    return 1023 - (int)((uint32_t)__builtin_bit_cast(uint64_t, d) & 0x3FFu);
}
__device__ __forceinline__ float route_ord_value(uint32_t ord) {
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ void dce(double& a, double& b) {
    const double x = a, y = b;
    a = __builtin_fmax(x, y);
    b = __builtin_fmin(x, y);
}

// Eight keys sorted descending: Batcher's odd-even merge sort (19 exchanges).
__device__ __forceinline__ void dsort8(double* k) {
#pragma unroll
    for (int p = 1; p < 8; p <<= 1)
#pragma unroll
        for (int q = p; q >= 1; q >>= 1)
#pragma unroll
            for (int j = q % p; j <= 7 - q; j += 2 * q)
#pragma unroll
                for (int i = 0; i <= (q - 1 < 7 - j - q ? q - 1 : 7 - j - q); ++i)
                    if ((i + j) / (2 * p) == (i + j + q) / (2 * p)) dce(k[i + j], k[i + j + q]);
}

// The eight largest of two descending runs of eight, descending: the
// elementwise max of a and b reversed holds exactly the top eight of the
// union as a bitonic sequence, which three half-cleaner stages sort.
__device__ __forceinline__ void dmerge8(double* a, const double* b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmax(a[i], b[7 - i]);
#pragma unroll
    for (int s = 4; s >= 1; s >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & s) == 0) dce(a[i], a[i + s]);
}

template <int CTRL>
__device__ __forceinline__ double dpp_dkey(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Eight lanes per token row, for 128 < E <= 256 and k <= 8.  Lane p of a
// group holds the 32 logits 32j + 4p + c (j < 8, c < 4): each of its eight
// 16-byte loads is one eighth of a 128-byte run of the row that the group
// reads whole.  The lane sorts its keys in four runs of eight and merges them
// down to its top eight; three exchanges across the group (DPP xor 1, xor 2,
// mirror within 8) each merge a lane's top eight with a partner's holding the
// other half of the candidates, after which every lane of the group holds
// the row's top eight in order.  Lane p keeps slot p.
template <bool FULL>
__global__ __launch_bounds__(256) void topk_merge_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                         int k, int32_t* __restrict__ ids, float* __restrict__ w,
                                                         int32_t* __restrict__ rec, int64_t rec_stride,
                                                         int64_t s0) {
    const int p = threadIdx.x & 7;
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 3) + (threadIdx.x >> 3);
    // every lane takes part in the exchanges; rows past T compute on row 0 and store nothing
    const bool live = row < T;
    const float* src = logits + (live ? row : 0) * E;
    double g[32];
    if (FULL) {
        // E == 256: every lane's 32 candidates are in the row
        float4 q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = *reinterpret_cast<const float4*>(src + 32 * j + 4 * p);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = 32 * j + 4 * p;
            g[4 * j] = route_dkey(q[j].x, e);
            g[4 * j + 1] = route_dkey(q[j].y, e + 1);
            g[4 * j + 2] = route_dkey(q[j].z, e + 2);
            g[4 * j + 3] = route_dkey(q[j].w, e + 3);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const int e = 32 * (r >> 2) + 4 * p + (r & 3);
            const int ec = e < E ? e : E - 1;
            const uint64_t b = __builtin_bit_cast(uint64_t, route_dkey(src[ec], ec));
            g[r] = __builtin_bit_cast(double, e < E ? b : 0ull);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) dsort8(g + 8 * r);
    dmerge8(g, g + 8);
    dmerge8(g + 16, g + 24);
    dmerge8(g, g + 16);
    double o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = dpp_dkey<0xB1>(g[i]);  // lane xor 1
    dmerge8(g, o);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = dpp_dkey<0x4E>(g[i]);  // lane xor 2
    dmerge8(g, o);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = dpp_dkey<0x141>(g[i]);  // lane 7 - p
    dmerge8(g, o);
    double mine = g[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mine = p == i ? g[i] : mine;
    const float m = route_ord_value(route_dkey_ord(g[0]));
    const float my_val = route_ord_value(route_dkey_ord(mine));
    const float ex = p < k ? expf(my_val - m) : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float o2 = __shfl(ex, j, 8);
        if (j < k) sum += o2;
    }
    if (live && p < k) {
        const int my_id = route_dkey_id(mine);
        ids[row * k + p] = my_id;
        w[row * k + p] = ex / sum;
        if (rec) rec[(int64_t)p * rec_stride + s0 + row] = my_id;
    }
}

// One thread per token: read the k recorded ids (coalesced along the sequence
// for each slot), validate, gather the k logits, softmax.
__global__ __launch_bounds__(256) void replay_kernel(const int32_t* __restrict__ rec, int k, int64_t S,
                                                     int64_t s0, int64_t T, const float* __restrict__ logits,
                                                     int E, int32_t* __restrict__ ids, float* __restrict__ w,
                                                     int32_t* __restrict__ status) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    int id[MAXK];
    bool bad = false, dup = false;
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
        if (j < k) {
            id[j] = rec[(int64_t)j * S + s0 + t];
            bad |= (id[j] < 0) | (id[j] >= E);
        }
    }
#pragma unroll
    for (int j = 1; j < MAXK; ++j)
#pragma unroll
        for (int i = 0; i < MAXK; ++i)
            if (i < j && j < k) dup |= id[i] == id[j];
    float g[MAXK];
    float m = -INFINITY;
    if (!bad) {
#pragma unroll
        for (int j = 0; j < MAXK; ++j)
            if (j < k) {
                g[j] = logits[t * E + id[j]];
                m = fmaxf(m, g[j]);
            }
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; ++j)
        if (j < k) {
            g[j] = bad ? 0.f : expf(g[j] - m);
            sum += g[j];
        }
#pragma unroll
    for (int j = 0; j < MAXK; ++j)
        if (j < k) {
            ids[t * k + j] = id[j];
            w[t * k + j] = bad ? 0.f : g[j] / sum;
        }
    int flags = (bad ? MOE_FLAG_BAD_ID : 0) | (dup ? MOE_FLAG_DUP_ID : 0);
    if (flags && status) atomicOr(status, flags);
}

// One wave per token row of d_logits: the token's k slots are uniform loads,
// each slot's contribution w_j (g_j - <w, g>) is formed once, and every lane
// writes its elements of the row (64 consecutive floats per store), each the
// sum of the contributions whose slot holds that id, in slot order (a
// repeated id sums its slots).
template <bool PARTS>
__global__ __launch_bounds__(256) void gate_backward_kernel(const float* __restrict__ d_gate_in,
                                                            const float* __restrict__ part,
                                                            const int32_t* __restrict__ pair_row, int ngroups,
                                                            const float* __restrict__ w,
                                                            const int32_t* __restrict__ ids, int64_t T,
                                                            int k, int E, float* __restrict__ d_gate_out,
                                                            float* __restrict__ d_logits) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    float dg[MAXK];
    if constexpr (PARTS) {
        // four slots at a time: lanes 16q .. 16q + 15 sum the group partials
        // of slot 4*it + q (a fixed butterfly order), read back uniformly
#pragma unroll
        for (int it = 0; it < MAXK / 4; ++it) {
            if (4 * it < k) {
                const int j = 4 * it + (lane >> 4), g = lane & 15;
                float v = 0.f;
                if (j < k && g < ngroups) {
                    const int r = pair_row[t * k + j];
                    if (r >= 0) v = part[(int64_t)r * MOE_GATE_PARTS + g];
                }
                v = group_sum<16>(v);
#pragma unroll
                for (int q = 0; q < 4; ++q) dg[4 * it + q] = __shfl(v, 16 * q);
                const float mine = __shfl(v, 16 * (lane & 3));
                if ((lane >> 2) == it && lane < k) d_gate_out[t * k + lane] = mine;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) dg[4 * it + q] = 0.f;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < MAXK; ++j) dg[j] = j < k ? d_gate_in[t * k + j] : 0.f;
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; ++j)
        if (j < k) dot += w[t * k + j] * dg[j];
    int id[MAXK];
    float c[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
        id[j] = j < k ? ids[t * k + j] : -1;
        c[j] = j < k ? w[t * k + j] * (dg[j] - dot) : 0.f;
    }
    float* out = d_logits + t * E;
    for (int e = lane; e < E; e += 64) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < MAXK; ++j)
            if (id[j] == e) acc += c[j];
        out[e] = acc;
    }
}

}  // namespace moe

using namespace moe;

static int launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                       int32_t* rec, int64_t rec_stride, int64_t s0, hipStream_t stream) {
    if (T == 0) return MOE_OK;
    if (E <= 256) {
        dim3 grid16((unsigned)((T + 15) / 16)), block16(256);
        const int vpl = (E + 15) / 16;
        auto go = [&](auto kern) {
            kern<<<grid16, block16, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
        };
        if (vpl <= 1)
            go(topk16_kernel<1, 1>);
        else if (vpl <= 2)
            go(topk16_kernel<2, 2>);
        else if (vpl <= 4)
            go(topk16_kernel<4, 4>);
        else if (vpl <= 8)
            go(topk16_kernel<8, 8>);
        else if (k <= 8) {
            dim3 grid8((unsigned)((T + 31) / 32));
            if (E == 256)
                topk_merge_kernel<true><<<grid8, block16, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
            else
                topk_merge_kernel<false><<<grid8, block16, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
        }
        else
            go(topk16_kernel<16, 16>);
        MOE_LAUNCH_CHECK("topk16_kernel");
        return MOE_OK;
    }
    const int waves_per_block = 4;
    dim3 grid((unsigned)((T + waves_per_block - 1) / waves_per_block)), block(64 * waves_per_block);
    int vpl = (E + 63) / 64;
    if (vpl <= 1)
        topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
    else if (vpl <= 2)
        topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
    else if (vpl <= 4)
        topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
    else if (vpl <= 8)
        topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
    else
        topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, w, rec, rec_stride, s0);
    MOE_LAUNCH_CHECK("topk_kernel");
    return MOE_OK;
}

static int check_topk_args(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w) {
    // up to 2^33 rows: every launch shape (at least 4 rows per workgroup)
    // stays within the 2^31 - 1 workgroups of a grid dimension
    MOE_REQUIRE(T >= 0 && T <= (int64_t)1 << 33, MOE_ERR_SHAPE, "route_topk: bad T=%lld", (long long)T);
    MOE_REQUIRE(E >= 1 && E <= 1024, MOE_ERR_SHAPE, "route_topk: E=%d outside [1, 1024]", E);
    MOE_REQUIRE(k >= 1 && k <= MAXK && k <= E, MOE_ERR_SHAPE, "route_topk: k=%d outside [1, min(16, E)]", k);
    MOE_REQUIRE(T == 0 || (logits && ids && w), MOE_ERR_NULL, "route_topk: NULL logits/ids/w");
    return MOE_OK;
}

extern "C" int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w,
                              hipStream_t stream) {
    int rc = check_topk_args(logits, T, E, k, ids, w);
    if (rc) return rc;
    return launch_topk(logits, T, E, k, ids, w, nullptr, 0, 0, stream);
}

extern "C" int moe_route_topk_capture(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                                      float* w, int32_t* rec, int32_t n_layers, int64_t seq_len, int32_t layer,
                                      int64_t s0, hipStream_t stream) {
    int rc = check_topk_args(logits, T, E, k, ids, w);
    if (rc) return rc;
    MOE_REQUIRE(rec, MOE_ERR_NULL, "route_topk_capture: NULL record");
    MOE_REQUIRE(n_layers >= 1 && layer >= 0 && layer < n_layers, MOE_ERR_SHAPE,
                "route_topk_capture: layer %d outside [0, %d)", layer, n_layers);
    MOE_REQUIRE(s0 >= 0 && seq_len >= 0 && s0 + T <= seq_len, MOE_ERR_SHAPE,
                "route_topk_capture: tokens [%lld, %lld) outside seq_len %lld", (long long)s0,
                (long long)(s0 + T), (long long)seq_len);
    return launch_topk(logits, T, E, k, ids, w, rec + (int64_t)layer * k * seq_len, seq_len, s0, stream);
}

extern "C" int moe_replay_load(const int32_t* rec, int32_t n_layers, int32_t k, int64_t seq_len, int32_t layer,
                               int64_t s0, int64_t T, const float* logits, int32_t E, int32_t* ids, float* w,
                               int32_t* dev_status, hipStream_t stream) {
    MOE_REQUIRE(k >= 1 && k <= MAXK, MOE_ERR_SHAPE, "replay_load: k=%d outside [1, 16]", k);
    MOE_REQUIRE(E >= 1 && E <= 1024, MOE_ERR_SHAPE, "replay_load: E=%d outside [1, 1024]", E);
    MOE_REQUIRE(n_layers >= 1 && layer >= 0 && layer < n_layers, MOE_ERR_SHAPE,
                "replay_load: layer %d outside [0, %d)", layer, n_layers);
    MOE_REQUIRE(T >= 0 && s0 >= 0 && seq_len >= 0 && s0 + T <= seq_len, MOE_ERR_SHAPE,
                "replay_load: tokens [%lld, %lld) outside seq_len %lld", (long long)s0, (long long)(s0 + T),
                (long long)seq_len);
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(rec && logits && ids && w, MOE_ERR_NULL, "replay_load: NULL rec/logits/ids/w");
    const int64_t S = seq_len;
    // one wave per block: a 16384-token chunk spreads over 256 CUs, not 64
    dim3 block(64), grid((unsigned)((T + 63) / 64));
    replay_kernel<<<grid, block, 0, stream>>>(rec + (int64_t)layer * k * S, k, S, s0, T, logits, E, ids, w,
                                              dev_status);
    MOE_LAUNCH_CHECK("replay_kernel");
    return MOE_OK;
}

extern "C" int moe_gate_backward(const float* d_gate, const float* w, const int32_t* ids, int64_t T, int32_t k,
                                 int32_t E, float* d_logits, hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && E >= 1 && E <= 1024, MOE_ERR_SHAPE,
                "gate_backward: bad T/k/E");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(d_gate && w && ids && d_logits, MOE_ERR_NULL, "gate_backward: NULL argument");
    gate_backward_kernel<false><<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(
        d_gate, nullptr, nullptr, 0, w, ids, T, k, E, nullptr, d_logits);
    MOE_LAUNCH_CHECK("gate_backward_kernel");
    return MOE_OK;
}

extern "C" int moe_gate_backward_parts(const float* gate_part, const int32_t* pair_row, int64_t row_cap, int32_t d,
                                       const float* w, const int32_t* ids, int64_t T, int32_t k, int32_t E,
                                       float* d_gate, float* d_logits, hipStream_t stream) {
    MOE_REQUIRE(T >= 0 && k >= 1 && k <= MAXK && E >= 1 && E <= 1024, MOE_ERR_SHAPE,
                "gate_backward_parts: bad T/k/E");
    MOE_REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "gate_backward_parts: d=%d must be a multiple of 128", d);
    MOE_REQUIRE(row_cap >= 0, MOE_ERR_SHAPE, "gate_backward_parts: bad row_cap");
    if (T == 0) return MOE_OK;
    MOE_REQUIRE(pair_row && w && ids && d_gate && d_logits && (row_cap == 0 || gate_part), MOE_ERR_NULL,
                "gate_backward_parts: NULL argument");
    gate_backward_kernel<true><<<dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream>>>(
        nullptr, gate_part, pair_row, gate_groups(d), w, ids, T, k, E, d_gate, d_logits);
    MOE_LAUNCH_CHECK("gate_backward_kernel");
    return MOE_OK;
}
