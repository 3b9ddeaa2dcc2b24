// Shared device helpers and host-side error plumbing for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

// Workgroups are dealt to the chip's 8 XCDs in turn (workgroup i to XCD i % 8).
// For a grid of n tiles with n % 8 == 0, the tile that workgroup bid takes so
// that XCD x runs the x-th contiguous eighth of the tiles in order: tiles that
// are neighbours in memory then run side by side in one XCD (and its L2)
// rather than spread over all eight.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t n) {
    return (n & 7) ? bid : (bid & 7) * (n >> 3) + (bid >> 3);
}

// ---------------------------------------------------------------- host side
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int num_cus();  // compute units of the current device (cached per device)

#define MOE_REQUIRE(cond, code, ...)                 \
    do {                                             \
        if (!(cond)) return ::moe::fail(code, __VA_ARGS__); \
    } while (0)

#define MOE_LAUNCH_CHECK(what)                                                         \
    do {                                                                               \
        hipError_t e_ = hipGetLastError();                                             \
        if (e_ != hipSuccess)                                                          \
            return ::moe::fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e_));   \
    } while (0)

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}
// The same rounding (nearest even) in one instruction: gfx950's
// v_cvt_pk_bf16_f32, reached through a __bf16 vector conversion.  Only NaN
// payloads may differ from f32_to_bf16.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------- e4m3
constexpr float E4M3_MAX = 448.0f;
constexpr float QUANT_EPS = 9.094947017729282e-13f;  // 2^-40

// Round two fp32 values to OCP e4m3 (round to nearest even, saturating at
// +-448) and pack them into bytes 0,1 (HI = false) or 2,3 of `old`.
// v_cvt_pk_fp8_f32 rounds to nearest even on gfx950 (OCP format); the clamp
// gives the satfinite behaviour because the instruction itself would produce
// NaN past the largest finite value.
template <bool HI = false>
__device__ __forceinline__ int cvt_e4m3x2(float a, float b, int old = 0) {
    a = __builtin_amdgcn_fmed3f(a, -E4M3_MAX, E4M3_MAX);
    b = __builtin_amdgcn_fmed3f(b, -E4M3_MAX, E4M3_MAX);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    int w = cvt_e4m3x2<false>(a, b, 0);
    w = cvt_e4m3x2<true>(c, d, w);
    return (uint32_t)w;
}

// Scale pair of one quantisation tile from its absolute maximum: inv = 448/a,
// s = a/448 with a = max(amax, 2^-40); both divisions correctly rounded (the
// library is built without fast-math, so '/' is IEEE division).
struct TileScale {
    float inv, s;
};
__device__ __forceinline__ TileScale tile_scale(float amax) {
    float a = fmaxf(amax, QUANT_EPS);
    TileScale t;
    t.inv = E4M3_MAX / a;
    t.s = a / E4M3_MAX;
    return t;
}

// Power-of-two (UE8M0) variant: s = 2^e with e the smallest integer such that
// a <= 448 * 2^e.  Writing a = m * 2^E with m in [0.5, 1) (a >= 2^-40 is a
// normal float: E = biased exponent - 126, m <= 0.875 exactly when the
// mantissa field is <= 0x600000) and 448 = 0.875 * 2^9 gives e = E - 9 when
// m <= 0.875, else E - 8.  s and inv = 2^-e are built from their bits (exact).
__device__ __forceinline__ TileScale tile_scale_pow2(float amax) {
    const uint32_t u = __float_as_uint(fmaxf(amax, QUANT_EPS));
    const int E = (int)((u >> 23) & 0xFFu) - 126;
    const int e = (u & 0x7FFFFFu) <= 0x600000u ? E - 9 : E - 8;
    TileScale t;
    t.s = __uint_as_float((uint32_t)(e + 127) << 23);
    t.inv = __uint_as_float((uint32_t)(127 - e) << 23);
    return t;
}
template <bool POW2>
__device__ __forceinline__ TileScale tile_scale_t(float amax) {
    if constexpr (POW2) return tile_scale_pow2(amax);
    else return tile_scale(amax);
}
// E8M0 code of a power-of-two fp32 scale (its biased exponent field)
__device__ __forceinline__ int e8m0_of(float pow2) { return (int)((__float_as_uint(pow2) >> 23) & 0xFFu); }

// ---------------------------------------------------------------- SwiGLU
// sigmoid and silu with the hardware exp2 and reciprocal (about 1 ulp each);
// exp2 overflows to inf for x below about -88, which gives sigmoid = 0
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
__device__ __forceinline__ float silu(float x) { return x * sigmoid_fast(x); }

// ---------------------------------------------------------------- wave reductions
// xor-butterfly max over groups of `width` lanes (width a power of two <= 64)
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WIDTH));
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WIDTH);
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace moe
