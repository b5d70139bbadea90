// Wavefront-level helpers shared by the decode kernels: cross-row swaps and reductions (gfx950 row permutes and
// DPP), ordering of LDS exchanges inside a single-wavefront workgroup, global-to-LDS DMA loads and explicit waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Cross-row reductions over the four 16-lane rows of a wavefront with the gfx950 row swaps. Two compiler traps
// are avoided here: the second operand goes through an empty asm statement (a swap whose operands the compiler
// can prove equal is folded into the identity), and the result pair is copied into named integers before use
// (reading element 1 of the pair through a bit cast was lowered as element 0).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ void swap16(uint32_t u, uint32_t &a, uint32_t &b) {
    auto p = __builtin_amdgcn_permlane16_swap(u, opaque(u), false, false);   // rows (0,1) and (2,3)
    a = p[0];
    b = p[1];
}
__device__ __forceinline__ void swap32(uint32_t u, uint32_t &a, uint32_t &b) {
    auto p = __builtin_amdgcn_permlane32_swap(u, opaque(u), false, false);   // halves (0,1) and (2,3)
    a = p[0];
    b = p[1];
}
__device__ __forceinline__ float rows_max(float v) {
    uint32_t a, b;
    swap16(__builtin_bit_cast(uint32_t, v), a, b);
    v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
    swap32(__builtin_bit_cast(uint32_t, v), a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float rows_sum(float v) {
    uint32_t a, b;
    swap16(__builtin_bit_cast(uint32_t, v), a, b);
    v = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
    swap32(__builtin_bit_cast(uint32_t, v), a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Sum over the 16 lanes of each row with DPP lane permutations (every lane of the row ends with the same value:
// each step adds a lane and its mirror, an exchange that gives both the same rounded sum).
template <int CTRL>
__device__ __forceinline__ float dpp_xadd(float v) {
    const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return v + __builtin_bit_cast(float, s);
}
constexpr int DPP_QUAD_1032 = 0xB1;      // quad_perm [1, 0, 3, 2]: lane pairs (0,1), (2,3)
constexpr int DPP_QUAD_2301 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_xadd<DPP_QUAD_1032>(v);
    v = dpp_xadd<DPP_QUAD_2301>(v);
    v = dpp_xadd<DPP_ROW_HALF_MIRROR>(v);
    return dpp_xadd<DPP_ROW_MIRROR>(v);
}

template <int CTRL>
__device__ __forceinline__ float dpp_xmax(float v) {
    const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, s));
}
__device__ __forceinline__ float row16_max(float v) {
    v = dpp_xmax<DPP_QUAD_1032>(v);
    v = dpp_xmax<DPP_QUAD_2301>(v);
    v = dpp_xmax<DPP_ROW_HALF_MIRROR>(v);
    return dpp_xmax<DPP_ROW_MIRROR>(v);
}

// Bitwise OR with the value of another lane of the same 16-lane row (DPP), and over each lane quad
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_xor_or(uint32_t v) {
    return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_ROW_ROR8 = 0x128;   // row_ror:8: lane i reads lane (i + 8) % 16 of its row
__device__ __forceinline__ uint32_t quad_or(uint32_t v) {
    return dpp_xor_or<DPP_QUAD_2301>(dpp_xor_or<DPP_QUAD_1032>(v));
}

// Cross-lane exchange through LDS inside one wavefront (every workgroup of the decode kernel is a single
// wavefront). LDS operations are performed in one order per CU and complete in a wavefront's execution order, so a
// read issued after a write sees it without draining the LDS counter first; only the compiler must not reorder them.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" : : : "memory"); }

// LDS-DMA load: 16 bytes per lane from `src` into LDS at lds_base + 16 * lane (lds_base goes through M0, which
// the statement saves and restores). Issued from inline asm so that the compiler's wait insertion, which cannot tell
// the destination from the other LDS buffers, does not drain the vector-memory counter before every LDS access; the
// destination's readers wait explicitly (wait_vmcnt), and loads complete in order, so these extra loads can only
// make the compiler's own counted waits stricter. Every caller streams data that a decode call reads once, so the
// load carries the non-temporal hint (a plain streaming read of HBM runs at 6.0-6.2 TB/s on MI355X, with
// non-temporal loads at 6.9-7.1 TB/s).
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}
// The same with a uniform base address in scalar registers and a 32-bit per-lane byte offset (the global
// scalar-base form: no per-lane 64-bit address arithmetic), for packed tile records, also with the non-temporal
// hint.
__device__ __forceinline__ void lds_dma16_s(uint64_t base, uint32_t lane_off, uint32_t lds_base) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(lane_off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

}  // namespace kvq
