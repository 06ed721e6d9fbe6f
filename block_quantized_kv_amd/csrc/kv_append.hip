// kv_append.hip -- quantize-on-append and dequant kernels for gfx950.
//
// Quantizer (den_llama.cpp, "What this fork is": Q4_G64 = signed INT4 + one
// FP16 scale per 64 values, byte-identical to the CPU reference; the q8_0 and
// q4_0 scale rules of the workload statement):
//   amax = max|x| over the group (exact), d = amax / Qmax (IEEE binary32
//   divide), d16 = binary16 nearest-even of min(d, 65504), dq = (float)d16,
//   q = clamp(rint(x / dq), -Qmax-1, Qmax) with an IEEE divide, 0 if dq == 0.
// One thread owns 8 consecutive channels of one row; a group is G/8 adjacent
// lanes that agree on amax through xor-shuffles.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

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

// Quantizes and stores this thread's 8 channels of one row of one plane.
template <int CODEC, int ROLE>
__device__ __forceinline__ void append_plane(const PlaneView &pl, const float *xsrc,
                                             const int32_t *seq_idx, const int64_t *pos_arr,
                                             int n_tokens, int32_t *dev_status, int64_t tid) {
    const int d = pl.head_dim;
    const int chunks = d / 8;  // threads per row
    const int64_t n_rows = (int64_t)n_tokens * pl.n_kv_heads;
    // Threads past the end still take part in the shuffles below (a group is
    // always inside one wave because G/8 divides 64 and d/8).
    const bool live = tid < n_rows * chunks;
    const int64_t row = live ? tid / chunks : 0;
    const int chunk = (int)(tid % chunks);
    const int tok = (int)(row / pl.n_kv_heads);
    const int head = (int)(row % pl.n_kv_heads);
    // destination first: its loads overlap the row's
    const int32_t sq = live ? seq_idx[tok] : 0;
    const int64_t pos = live ? pos_arr[tok] : 0;

    float x[8];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(xsrc + row * d + chunk * 8);
        const float4 v0 = src[0], v1 = src[1];
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
        for (int s = 0; s < 8; ++s) x[s] = 0.0f;
    }
    float amax = 0.0f;
    for (int s = 0; s < 8; ++s) amax = fmaxf(amax, fabsf(x[s]));
    constexpr int lanes_per_group = group_size(CODEC) / 8;
    for (int m = 1; m < lanes_per_group; m <<= 1) amax = fmaxf(amax, shfl_xor(amax, m));

    float dscale = __fdiv_rn(amax, (float)qmax(CODEC));
    dscale = fminf(dscale, 65504.0f);
    const _Float16 d16 = (_Float16)dscale;  // v_cvt_f16_f32: round to nearest even
    const float dq = (float)d16;
    int q[8];
    for (int s = 0; s < 8; ++s) {
        float r = dq == 0.0f ? 0.0f : __builtin_rintf(__fdiv_rn(x[s], dq));
        r = fminf(fmaxf(r, (float)(-qmax(CODEC) - 1)), (float)qmax(CODEC));
        q[s] = (int)r;
    }
    if (!live) return;
    if (sq < 0 || sq >= pl.n_seqs || pos < 0 || pos >= pl.capacity) {
        if (dev_status) *dev_status = 3;  // KVQ_ERANGE
        return;
    }
    const int64_t blk_idx = pos / kBlockRows;
    const int j = (int)(pos % kBlockRows);
    const int64_t head_lin = (int64_t)sq * pl.n_kv_heads + head;
    uint8_t *blk = pl.codes + head_lin * pl.head_code_stride + blk_idx * block_code_bytes(CODEC, d);
    uint16_t *sblk = pl.scales + head_lin * pl.head_scale_stride + blk_idx * block_scales(CODEC, d);
    store_codes<CODEC, ROLE>(blk, d, j, chunk * 8, q);
    if (chunk % lanes_per_group == 0) {
        const int g = chunk / lanes_per_group;
        const int si = ROLE == ROLE_K ? k_scale_index(CODEC, d, j, g) : v_scale_index(CODEC, d, j, g);
        sblk[si] = __builtin_bit_cast(uint16_t, d16);
    }
}

// grid.y = 0: K plane, 1: V plane (one launch appends both).
template <int KC, int VC>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.y == 0) {
        if (a.x[0]) append_plane<KC, ROLE_K>(a.plane[0], a.x[0], a.seq_idx, a.pos, a.n_tokens,
                                             a.dev_status, tid);
    } else {
        if (a.x[1]) append_plane<VC, ROLE_V>(a.plane[1], a.x[1], a.seq_idx, a.pos, a.n_tokens,
                                             a.dev_status, tid);
    }
}

template <int CODEC, int ROLE>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
    const int d = a.plane.head_dim;
    const int chunks = d / 8;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)a.plane.n_kv_heads * a.n_rows * chunks;
    if (tid >= total) return;
    const int chunk = (int)(tid % chunks);
    const int64_t r = (tid / chunks) % a.n_rows;
    const int head = (int)(tid / chunks / a.n_rows);
    const int64_t pos = a.row0 + r;
    const int64_t blk_idx = pos / kBlockRows;
    const int j = (int)(pos % kBlockRows);
    const int64_t head_lin = (int64_t)a.seq * a.plane.n_kv_heads + head;
    const uint8_t *blk = a.plane.codes + head_lin * a.plane.head_code_stride +
                         blk_idx * block_code_bytes(CODEC, d);
    const uint16_t *sblk = a.plane.scales + head_lin * a.plane.head_scale_stride +
                           blk_idx * block_scales(CODEC, d);
    float o[8];
    for (int s = 0; s < 8; ++s) {
        const int c = chunk * 8 + s;
        const CodePos p = ROLE == ROLE_K ? k_code_pos(CODEC, d, j, c) : v_code_pos(CODEC, d, j, c);
        int qi;
        if constexpr (is8(CODEC)) {
            qi = (int8_t)blk[p.byte];
        } else {
            const int nib = (blk[p.byte] >> p.shift) & 0xF;
            qi = CODEC == Q4_0 ? nib - 8 : (nib >= 8 ? nib - 16 : nib);
        }
        const int g = c / group_size(CODEC);
        const int si = ROLE == ROLE_K ? k_scale_index(CODEC, d, j, g) : v_scale_index(CODEC, d, j, g);
        const float dq = (float)__builtin_bit_cast(_Float16, sblk[si]);
        o[s] = (float)qi * dq;  // exact
    }
    float4 *dst = reinterpret_cast<float4 *>(a.out + ((int64_t)head * a.n_rows + r) * d + chunk * 8);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
    const int64_t threads =
        (int64_t)a.n_tokens * a.plane[0].n_kv_heads * (a.plane[0].head_dim / 8);
    if (threads == 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((threads + 255) / 256), 2);
    switch (a.plane[0].codec * 3 + a.plane[1].codec) {
        case Q8_0 * 3 + Q8_0: append_kernel<Q8_0, Q8_0><<<grid, block, 0, s>>>(a); break;
        case Q8_0 * 3 + Q4_0: append_kernel<Q8_0, Q4_0><<<grid, block, 0, s>>>(a); break;
        case Q8_0 * 3 + Q4_G64: append_kernel<Q8_0, Q4_G64><<<grid, block, 0, s>>>(a); break;
        case Q4_0 * 3 + Q8_0: append_kernel<Q4_0, Q8_0><<<grid, block, 0, s>>>(a); break;
        case Q4_0 * 3 + Q4_0: append_kernel<Q4_0, Q4_0><<<grid, block, 0, s>>>(a); break;
        case Q4_0 * 3 + Q4_G64: append_kernel<Q4_0, Q4_G64><<<grid, block, 0, s>>>(a); break;
        case Q4_G64 * 3 + Q8_0: append_kernel<Q4_G64, Q8_0><<<grid, block, 0, s>>>(a); break;
        case Q4_G64 * 3 + Q4_0: append_kernel<Q4_G64, Q4_0><<<grid, block, 0, s>>>(a); break;
        case Q4_G64 * 3 + Q4_G64: append_kernel<Q4_G64, Q4_G64><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs &a, hipStream_t s) {
    const int64_t threads = (int64_t)a.plane.n_kv_heads * a.n_rows * (a.plane.head_dim / 8);
    if (threads == 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((threads + 255) / 256));
    switch (a.plane.codec * 2 + a.role) {
        case Q8_0 * 2 + ROLE_K: dequant_kernel<Q8_0, ROLE_K><<<grid, block, 0, s>>>(a); break;
        case Q8_0 * 2 + ROLE_V: dequant_kernel<Q8_0, ROLE_V><<<grid, block, 0, s>>>(a); break;
        case Q4_0 * 2 + ROLE_K: dequant_kernel<Q4_0, ROLE_K><<<grid, block, 0, s>>>(a); break;
        case Q4_0 * 2 + ROLE_V: dequant_kernel<Q4_0, ROLE_V><<<grid, block, 0, s>>>(a); break;
        case Q4_G64 * 2 + ROLE_K: dequant_kernel<Q4_G64, ROLE_K><<<grid, block, 0, s>>>(a); break;
        case Q4_G64 * 2 + ROLE_V: dequant_kernel<Q4_G64, ROLE_V><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
