// kv_append.hip -- quantize-on-append and dequant kernels for gfx950.
//
// Quantizer (den_llama.cpp, "What this fork is": Q4_G64 = signed INT4 + one
// FP16 scale per 64 values, byte-identical to the CPU reference; the q8_0 and
// q4_0 scale rules of the workload statement):
//   amax = max|x| over the group (exact), d = amax / Qmax (IEEE binary32
//   divide), d16 = binary16 nearest-even of min(d, 65504), dq = (float)d16,
//   q = clamp(rint(x / dq), -Qmax-1, Qmax) with an IEEE divide, 0 if dq == 0.
// One thread owns 8 consecutive channels of one row (kvq_quant.h).
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {

namespace {

// Quantizes and stores this thread's 8 channels of one row of one plane.
template <int CODEC, int ROLE>
__device__ __forceinline__ void append_plane(const PlaneView &pl, const PageTable &pt, const float *xsrc,
                                             const int32_t *seq_idx, const int64_t *pos_arr,
                                             int n_tokens, int32_t *dev_status, int64_t tid) {
    const int d = pl.head_dim;
    const int chunks = d / 8;  // threads per row
    const int64_t n_rows = (int64_t)n_tokens * pl.n_kv_heads;
    // Threads past the end still take part in the group shuffles (a group is
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
    const int n_seqs = pt.table ? pt.n_seqs : pl.n_seqs;
    const int64_t cap = pt.table ? (int64_t)pt.table_stride * pt.page_rows : pl.capacity;
    bool in_range = sq >= 0 && sq < n_seqs && pos >= 0 && pos < cap;
    int64_t head_lin = 0, prow = 0;
    if (live && in_range) in_range = phys_row(pl, pt, sq, head, pos, head_lin, prow);
    if (live && !in_range && dev_status) *dev_status = 3;  // KVQ_ERANGE
    quantize_store<CODEC, ROLE>(pl, head_lin, prow, chunk, x, live && in_range);
}

// grid.y = 0: K plane, 1: V plane (one launch appends both).
template <int KC, int VC>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.y == 0) {
        if (a.x[0]) append_plane<KC, ROLE_K>(a.plane[0], a.pt, a.x[0], a.seq_idx, a.pos, a.n_tokens,
                                             a.dev_status, tid);
    } else {
        if (a.x[1]) append_plane<VC, ROLE_V>(a.plane[1], a.pt, a.x[1], a.seq_idx, a.pos, a.n_tokens,
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
