// kvq_device.h -- device helpers shared by the gfx950 kernels: vector types,
// code unpacking into binary16 matrix-core operands, cross-lane reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_layout.h"

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
// Views for reading back LDS words that were stored as uint32_t: the
// may_alias attribute keeps the compiler from reordering (or hoisting out of
// a loop) such a read past the store under type-based alias rules.
typedef _Float16 f16_alias __attribute__((may_alias));
typedef _Float16 h2_alias __attribute__((ext_vector_type(2), may_alias));

__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ f4 mfma16x16x32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16x16x32_bf16(bf8 a, bf8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- 4-bit codes -------------------------------------------------------------
// A word holds 8 nibbles in slot order (nibble positions 0,4,1,5,2,6,3,7 for
// slots 0..7).  With the binary16 pattern 0x6400 (= 1024.0, unit fraction step)
// merged in, a nibble n in the low 4 fraction bits reads as 1024 + n and a
// nibble in fraction bits 4..7 reads as 1024 + 16 n; both are exact.
// n is the offset-8 code q + 8: q4_0 stores it; Q4_G64 stores q & 0xF
// (two's complement), and q + 8 = (q & 0xF) ^ 8.  One v_bitop3 per pair does
// mask, sign flip and merge: f(w, M, K) = M ? (w ^ K) : K with K holding the
// magic outside M and the flip bit inside it.
// Result: slots (0,1) = 1024+n, (2,3) = 1024+16n, (4,5) = 1024+n, (6,7) = 1024+16n.
template <int CODEC>
__device__ __forceinline__ u4 nib_magic(uint32_t w) {
    constexpr uint32_t flip = CODEC == Q4_G64 ? 0x8u : 0x0u;
    constexpr uint32_t M_LO = 0x000F000Fu, M_HI = 0x00F000F0u;
    constexpr uint32_t K_LO = 0x64006400u | (flip * 0x00010001u);
    constexpr uint32_t K_HI = 0x64006400u | (flip * 0x00100010u);
    const uint32_t w8 = w >> 8;
    u4 r;
    r.x = __builtin_amdgcn_bitop3_b32(w, M_LO, K_LO, 0x6A);
    r.y = __builtin_amdgcn_bitop3_b32(w, M_HI, K_HI, 0x6A);
    r.z = __builtin_amdgcn_bitop3_b32(w8, M_LO, K_LO, 0x6A);
    r.w = __builtin_amdgcn_bitop3_b32(w8, M_HI, K_HI, 0x6A);
    return r;
}

// ---- 8-bit codes -------------------------------------------------------------
// Byte b (two's complement) becomes binary16 1152 + b = 0x6400 | (b ^ 0x80).
__device__ __forceinline__ u2 byte_magic(uint32_t w) {
    const uint32_t x = w ^ 0x80808080u;
    u2 r;
    r.x = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);  // bytes b0, b1
    r.y = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);  // bytes b2, b3
    return r;
}

// K operand (A of S^T = K Q^T) for one k-step: 8 binary16 values that equal the
// code plus a known per-slot bias (removed through the accumulator init).
template <int CODEC>
__device__ __forceinline__ h8 k_operand(const uint32_t *w) {
    if constexpr (is16(CODEC)) {  // the stored binary16 values themselves
        const u4 r = {w[0], w[1], w[2], w[3]};
        return __builtin_bit_cast(h8, r);
    } else if constexpr (is8(CODEC)) {
        const u2 a = byte_magic(w[0]), b = byte_magic(w[1]);
        const u4 r = {a.x, a.y, b.x, b.y};
        return __builtin_bit_cast(h8, r);
    } else {
        return __builtin_bit_cast(h8, nib_magic<CODEC>(w[0]));
    }
}

// Bias of slot s in k_operand for code 0, and the factor the query must carry
// in that slot so that slot * factor = (code + bias) * query.
template <int CODEC>
__device__ __forceinline__ constexpr float k_slot_bias(int s) {
    return is16(CODEC) ? 0.0f : is8(CODEC) ? 1152.0f : (((s >> 1) & 1) ? 1152.0f : 1032.0f);
}
template <int CODEC>
__device__ __forceinline__ constexpr float k_slot_factor(int s) {
    return (is16(CODEC) || is8(CODEC)) ? 1.0f : (((s >> 1) & 1) ? 0.0625f : 1.0f);
}

// V operand (A of O^T = V^T P^T) for one 16-channel block: binary16 of
// code * dq (rounded to nearest even once; exact for subnormal scales), for the
// eight slot rows.  dq2[m] holds the scales of slots (2m, 2m+1).
template <int CODEC>
__device__ __forceinline__ h8 v_operand(const uint32_t *w, const h2_alias *dq2) {
    if constexpr (is16(CODEC)) {  // the stored binary16 values themselves (no scale)
        const u4 r = {w[0], w[1], w[2], w[3]};
        return __builtin_bit_cast(h8, r);
    }
    h2 v0, v1, v2, v3;
    if constexpr (is8(CODEC)) {
        const u2 a = byte_magic(w[0]), b = byte_magic(w[1]);
        const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
        v0 = (as_h2(a.x) + bias) * dq2[0];
        v1 = (as_h2(a.y) + bias) * dq2[1];
        v2 = (as_h2(b.x) + bias) * dq2[2];
        v3 = (as_h2(b.y) + bias) * dq2[3];
    } else {
        const u4 r = nib_magic<CODEC>(w[0]);
        const h2 b_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        const h2 b_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
        v0 = (as_h2(r.x) + b_lo) * dq2[0];
        v1 = (as_h2(r.y) * sixteenth + b_hi) * dq2[1];
        v2 = (as_h2(r.z) + b_lo) * dq2[2];
        v3 = (as_h2(r.w) * sixteenth + b_hi) * dq2[3];
    }
    h8 out;
    out.s01 = v0;
    out.s23 = v1;
    out.s45 = v2;
    out.s67 = v3;
    return out;
}

// ---- cross-lane ----------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Max / sum over the 4 lanes h, h+16, h+32, h+48 (every lane gets the result),
// on the vector ALU through gfx950's lane swaps: after a swap every lane holds
// its own value and its partner's (lane ^ 16, or lane ^ 32), in some order, so
// one max or add per stage gives all four lanes the same result with no trip
// through the LDS pipeline (measured about 1 % faster per decode step than
// ds_swizzle + ds_bpermute, whose waits also covered unrelated LDS reads).
// The halves are copied out of the result vector before the casts: a bit
// cast of a vector element reads element 0 in this compiler.
struct SwapPair {
    float a, b;
};
__device__ __forceinline__ SwapPair swap16(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a = p[0], b = p[1];
    return SwapPair{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}
__device__ __forceinline__ SwapPair swap32(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a = p[0], b = p[1];
    return SwapPair{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}
__device__ __forceinline__ float swap_max16(float v) {
    const SwapPair p = swap16(v);
    return __builtin_elementwise_maximum(p.a, p.b);
}
__device__ __forceinline__ float swap_max32(float v) {
    const SwapPair p = swap32(v);
    return __builtin_elementwise_maximum(p.a, p.b);
}
__device__ __forceinline__ float swap_sum16(float v) {
    const SwapPair p = swap16(v);
    return p.a + p.b;
}
__device__ __forceinline__ float swap_sum32(float v) {
    const SwapPair p = swap32(v);
    return p.a + p.b;
}

__device__ __forceinline__ float quad_max(float v) { return swap_max32(swap_max16(v)); }
__device__ __forceinline__ float quad_sum(float v) { return swap_sum32(swap_sum16(v)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Block gb of a paged sequence: its block-table index and its block within
// that page, for pages of pblk blocks (pblk >= 1).  A power-of-two page is a
// shift and a mask; otherwise one 32-bit division while the block index fits,
// and the 64-bit one beyond (a 64-bit division is a long scalar sequence with
// branches, and the scalar unit is shared by every wave of the compute unit).
struct PageSlot {
    int64_t entry;
    int within;
};
__device__ __forceinline__ PageSlot page_slot(int64_t gb, int pblk) {
    if ((pblk & (pblk - 1)) == 0) {
        const int sh = __builtin_ctz((unsigned)pblk);
        return PageSlot{gb >> sh, (int)(gb & (pblk - 1))};
    }
    if (gb >= 0 && gb <= 0xFFFFFFFFll) {
        const uint32_t g = (uint32_t)gb, q = g / (uint32_t)pblk;
        return PageSlot{(int64_t)q, (int)(g - q * (uint32_t)pblk)};
    }
    return PageSlot{gb / pblk, (int)(gb % pblk)};
}

}  // namespace kvq
