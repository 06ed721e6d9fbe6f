// kvq_quant.h -- quantize-on-append device code (den_llama.cpp, "What this
// fork is": Q4_G64 = signed INT4 + one FP16 scale per 64 values; q8_0 and
// q4_0, which the page names beside it, take the same rule at 32 values per
// group with Qmax 127 and 7), shared by the append kernel and the decode
// kernel's fused append.
//   amax = max|x| over the group (exact), d = amax / Qmax (IEEE binary32
//   divide), d16 = binary16 nearest-even of min(d, 65504), dq = (float)d16,
//   q = clamp(rint(x / dq), -Qmax-1, Qmax) with an IEEE divide, 0 if dq == 0.
// One thread owns 8 consecutive channels of one row; a group is G/8 adjacent
// lanes that agree on amax through xor-shuffles.
#pragma once
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// Writes the 8 codes q[0..7] of channels c0..c0+7 of block row j.
template <int CODEC, int ROLE>
__device__ __forceinline__ void store_codes(uint8_t *blk, int d, int j, int c0, const int *q) {
    if constexpr (ROLE == ROLE_K) {
        // The 8 channels are one k-step slot run of one lane: a single word
        // (4-bit) or two words (8-bit), written whole.
        const CodePos p0 = k_code_pos(CODEC, d, j, c0);
        if constexpr (is8(CODEC)) {
            uint32_t w0 = 0, w1 = 0;
            for (int s = 0; s < 4; ++s) w0 |= (uint32_t)(uint8_t)(int8_t)q[s] << (8 * s);
            for (int s = 0; s < 4; ++s) w1 |= (uint32_t)(uint8_t)(int8_t)q[4 + s] << (8 * s);
            *reinterpret_cast<u2 *>(blk + p0.byte) = u2{w0, w1};
        } else {
            uint32_t w = 0;
            for (int s = 0; s < 8; ++s) {
                const uint32_t nib = CODEC == Q4_0 ? (uint32_t)(q[s] + 8) : ((uint32_t)q[s] & 0xFu);
                w |= nib << (4 * slot_nibble(s));
            }
            *reinterpret_cast<uint32_t *>(blk + p0.byte) = w;
        }
    } else {
        // V role: each channel lives in a different lane word, shared with
        // seven other rows.  Bytes are stored directly; a nibble is replaced
        // with an atomic and (clear) followed by an atomic or (set) on its
        // word, which leave the other nibbles untouched whatever other threads
        // do to them (one thread's two atomics to one address stay in order).
        for (int s = 0; s < 8; ++s) {
            const CodePos p = v_code_pos(CODEC, d, j, c0 + s);
            if constexpr (is8(CODEC)) {
                blk[p.byte] = (uint8_t)(int8_t)q[s];
            } else {
                const uint32_t nib = CODEC == Q4_0 ? (uint32_t)(q[s] + 8) : ((uint32_t)q[s] & 0xFu);
                uint32_t *word = reinterpret_cast<uint32_t *>(blk + (p.byte & ~3));
                const int sh = 8 * (p.byte & 3) + p.shift;
                // clear then set this nibble; neither needs the old value back
                atomicAnd(word, ~(0xFu << sh));
                atomicOr(word, nib << sh);
            }
        }
    }
}

// Quantizes the 8 channels x[0..7] = channels 8*chunk .. 8*chunk+7 of row
// `pos` of head `head_lin` (= seq * n_kv_heads + kv-head) and stores codes and
// group scale.  Every lane of the wave must call it (the group maximum is
// shuffled between lanes); only lanes with `store` set write.
// The codes q[0..7] of this thread's 8 channels and the group's binary16
// scale.  Every lane of the wave must call it (the group maximum is shuffled
// between the group's G/8 adjacent lanes).
template <int CODEC>
__device__ __forceinline__ _Float16 quantize8(const float (&x)[8], int (&q)[8]) {
    float amax = 0.0f;
    for (int s = 0; s < 8; ++s) amax = fmaxf(amax, fabsf(x[s]));
    constexpr int lanes_per_group = group_size(CODEC) / 8;
    for (int m = 1; m < lanes_per_group; m <<= 1) amax = fmaxf(amax, shfl_xor(amax, m));
    float dscale = __fdiv_rn(amax, (float)qmax(CODEC));
    dscale = fminf(dscale, 65504.0f);
    const _Float16 d16 = (_Float16)dscale;  // v_cvt_f16_f32: round to nearest even
    const float dq = (float)d16;
    for (int s = 0; s < 8; ++s) {
        float r = dq == 0.0f ? 0.0f : __builtin_rintf(__fdiv_rn(x[s], dq));
        r = fminf(fmaxf(r, (float)(-qmax(CODEC) - 1)), (float)qmax(CODEC));
        q[s] = (int)r;
    }
    return d16;
}

// The f16 control codec: each value's binary16 nearest-even rounding
// (v_cvt_f16_f32), saturated at +-65504; no scales.  K role: the 8 values are
// one 16-byte slot run of one lane, stored whole; V role: each value is a
// 2-byte store of its own (no other row shares its bytes).
template <int ROLE>
__device__ __forceinline__ void store_f16(const PlaneView &pl, int64_t head_lin, int64_t pos, int chunk,
                                          const float (&x)[8]) {
    const int d = pl.head_dim;
    _Float16 h[8];
    for (int s = 0; s < 8; ++s) h[s] = (_Float16)fminf(fmaxf(x[s], -65504.0f), 65504.0f);
    const int j = (int)(pos % kBlockRows);
    uint8_t *blk = pl.codes + head_lin * pl.head_code_stride + (pos / kBlockRows) * block_code_bytes(F16, d);
    if constexpr (ROLE == ROLE_K) {
        u4 w;
        for (int m = 0; m < 4; ++m)
            w[m] = (uint32_t)__builtin_bit_cast(uint16_t, h[2 * m]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, h[2 * m + 1]) << 16);
        *reinterpret_cast<u4 *>(blk + k_code_pos(F16, d, j, chunk * 8).byte) = w;
    } else {
        for (int s = 0; s < 8; ++s)
            *reinterpret_cast<uint16_t *>(blk + v_code_pos(F16, d, j, chunk * 8 + s).byte) =
                __builtin_bit_cast(uint16_t, h[s]);
    }
}

template <int CODEC, int ROLE>
__device__ __forceinline__ void quantize_store(const PlaneView &pl, int64_t head_lin, int64_t pos, int chunk,
                                               const float (&x)[8], bool store) {
    if constexpr (is16(CODEC)) {
        if (store) store_f16<ROLE>(pl, head_lin, pos, chunk, x);
        return;
    }
    const int d = pl.head_dim;
    constexpr int lanes_per_group = group_size(CODEC) / 8;
    int q[8];
    const _Float16 d16 = quantize8<CODEC>(x, q);
    if (!store) return;
    const int64_t blk_idx = pos / kBlockRows;
    const int j = (int)(pos % kBlockRows);
    uint8_t *blk = pl.codes + head_lin * pl.head_code_stride + blk_idx * block_code_bytes(CODEC, d);
    uint16_t *sblk = pl.scales + head_lin * pl.head_scale_stride + blk_idx * block_scales(CODEC, d);
    store_codes<CODEC, ROLE>(blk, d, j, chunk * 8, q);
    if (chunk % lanes_per_group == 0) {
        const int g = chunk / lanes_per_group;
        const int si = ROLE == ROLE_K ? k_scale_index(CODEC, d, j, g) : v_scale_index(CODEC, d, j, g);
        sblk[si] = __builtin_bit_cast(uint16_t, d16);
    }
}

// Where row `pos` of sequence `seq`, kv-head `head` lives: head_lin indexes
// the planes' (sequence-or-page, kv-head) ranges, row the row inside it.
// Paged planes look the page up in the table (one load); false if the table
// sends the row outside the pool (nothing may be stored then).
__device__ __forceinline__ bool phys_row(const PlaneView &pl, const PageTable &pt, int64_t seq, int head, int64_t pos,
                                         int64_t &head_lin, int64_t &row) {
    if (!pt.table) {
        head_lin = seq * pl.n_kv_heads + head;
        row = pos;
        return true;
    }
    const int32_t page = pt.table[seq * pt.table_stride + pos / pt.page_rows];
    head_lin = (int64_t)page * pl.n_kv_heads + head;
    row = pos % pt.page_rows;
    return page >= 0 && page < pl.n_seqs;
}

}  // namespace kvq
