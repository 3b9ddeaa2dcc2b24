// MFMA and LDS helpers shared by the grouped GEMM kernels (gfx950).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) float* cfloat_ptr;


// 16- / 4-byte global -> LDS transfer (global_load_lds_dwordx4 / _dword): lane
// l's bytes land at LDS byte address m0 + l*size (m0 = `lds`, wave-uniform).
// Written as inline assembly so that the compiler does not know these VMEM
// instructions write LDS: it would otherwise wait for all of them (vmcnt(0))
// before every LDS read, serialising the pipeline.  Completion is awaited with
// explicit vmcnt waits followed by a barrier before a stage is read.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" : : "v"(g), "{m0}"(lds) : "memory");
}

// The same transfers with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset: the base advances by scalar adds along K, so no
// per-lane 64-bit address arithmetic is needed in the loop.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
// the same with the non-temporal hint, for operand bytes no other tile reads
__device__ __forceinline__ void dma16s_nt(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// s_waitcnt immediate waiting for vmcnt <= N only (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt immediate waiting for lgkmcnt == 0 only (LDS reads of this wave)
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

typedef const __attribute__((address_space(3))) u32x4* lds_u32x4_ptr;
typedef const __attribute__((address_space(3))) v2u* lds_v2u_ptr;
typedef const __attribute__((address_space(3))) uint32_t* lds_u32_ptr;
typedef const __attribute__((address_space(3))) uint8_t* lds_u8_ptr;

// Plain LDS loads (the compiler tracks their lgkmcnt).  `base` comes out of an
// opaque move placed after the stage's barrier, so no read can be hoisted
// above the barrier that makes the stage's DMA data visible.
template <int OFF>
__device__ __forceinline__ u32x4 lds16(uint32_t addr) {
    return *(lds_u32x4_ptr)(uintptr_t)(addr + OFF);
}
template <int OFF>
__device__ __forceinline__ v2u lds8(uint32_t addr) {
    return *(lds_v2u_ptr)(uintptr_t)(addr + OFF);
}
template <int OFF>
__device__ __forceinline__ uint32_t lds4(uint32_t addr) {
    return *(lds_u32_ptr)(uintptr_t)(addr + OFF);
}
template <int OFF>
__device__ __forceinline__ uint32_t lds1(uint32_t addr) {
    return *(lds_u8_ptr)(uintptr_t)(addr + OFF);
}
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}
// The same fence applied to a variable in place: later reads of `v` depend on
// this point, and no register copy is made (the copy opaque() needs costs a
// v_mov per address per use).
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }
// The same for a wave-uniform value kept in an SGPR: an address formed from it
// after this point cannot be hoisted out of the loop that contains it (per
// stage address pairs held across a loop cost a VGPR each).
__device__ __forceinline__ void pin_s(uint32_t& v) { asm volatile("" : "+s"(v)); }

// Workgroup barrier that the instruction scheduler may not move any
// instruction across: phases separated by it (MFMA work on one side, LDS reads
// on the other) stay where the source puts them.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ v8i join8(u32x4 lo, u32x4 hi) {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Cross-lane exchanges of gfx950 (no LDS): swap32 trades lanes 32..63 of `a`
// with lanes 0..31 of `b`; swap16 trades the odd 16-lane rows of `a` with the
// even rows of `b` (rows 1, 3 <-> 0, 2).
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // E8M0 127 = 2^0: the hardware block scales are 1, the fp32 scales are
    // applied by the caller
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}
// c + (2^(ea-127) 2^(eb-127)) * (a . b) with the E8M0 block scales applied by
// the matrix core: ea scales row (lane % 16) of a, eb row (lane % 16) of b
// (each lane passes the scale of the row whose K chunk it holds)
__device__ __forceinline__ v4f mfma16x16x128_e8m0(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}
// the same with a as packed fp4 e2m1 (32 values in the low 16 bytes of the
// lane's operand, element 2i in the low nibble of byte i) and b fp8 e4m3.
// Lane group g = lane / 16 of a holds K values [32g, 32g + 32) of its row; the
// fp8 operand's lane group g holds the 16-byte K chunks g and g + 4 (measured:
// with that layout the K indices of the two operands pair in order), and each
// lane's E8M0 scale covers exactly its own 32 values.
__device__ __forceinline__ v4f mfma16x16x128_fp4_e8m0(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, ea, 0, eb);
}

}  // namespace moe
