// kv_append.hip -- quantize-on-append and dequant kernels for gfx950.
//
// Quantizer (den_llama.cpp, "What this fork is": Q4_G64 = signed INT4 + one
// FP16 scale per 64 values, byte-identical to the CPU reference; q8_0 and
// q4_0, which the page names beside it, take the same rule at 32 values per
// group with Qmax 127 and 7):
//   amax = max|x| over the group (exact), d = amax / Qmax (IEEE binary32
//   divide), d16 = binary16 nearest-even of min(d, 65504), dq = (float)d16,
//   q = clamp(rint(x / dq), -Qmax-1, Qmax) with an IEEE divide, 0 if dq == 0.
// One thread owns 8 consecutive channels of one row (kvq_quant.h).
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {

namespace {

// Quantizes and stores the 8 channels `chunk` of token `tok`, kv-head `head`
// of one plane (live: the item exists; every lane of the wave calls it).
template <int CODEC, int ROLE>
__device__ __forceinline__ void append_one(const AppendArgs &a, const PlaneView &pl, const float *xsrc, int tok,
                                           int head, int chunk, bool live) {
    const int d = pl.head_dim;
    const int64_t row = (int64_t)tok * pl.n_kv_heads + head;
    // destination first: its loads overlap the row's
    const int32_t sq = live ? a.seq_idx[tok] : 0;
    const int64_t pos = live ? a.pos[tok] : 0;
    float x[8];
    if (live) {
        const float4 *src = reinterpret_cast<const float4 *>(xsrc + row * d + chunk * 8);
        const float4 v0 = src[0], v1 = src[1];
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
        for (int s = 0; s < 8; ++s) x[s] = 0.0f;
    }
    const int n_seqs = a.pt.table ? a.pt.n_seqs : pl.n_seqs;
    const int64_t cap = a.pt.table ? (int64_t)a.pt.table_stride * a.pt.page_rows : pl.capacity;
    bool in_range = sq >= 0 && sq < n_seqs && pos >= 0 && pos < cap;
    int64_t head_lin = 0, prow = 0;
    if (live && in_range) in_range = phys_row(pl, a.pt, sq, head, pos, head_lin, prow);
    if (live && !in_range && a.dev_status) *a.dev_status = 3;  // KVQ_ERANGE
    quantize_store<CODEC, ROLE>(pl, head_lin, prow, chunk, x, live && in_range);
}

// K plane: one thread per 8 channels of one (token, kv-head) row.  A K-role
// word belongs to one row, so every store is whole.
template <int KC>
__device__ __forceinline__ void append_k(const AppendArgs &a, int64_t tid) {
    const PlaneView &pl = a.plane[0];
    const int chunks = pl.head_dim / 8;  // threads per row
    const int64_t n_rows = (int64_t)a.n_tokens * pl.n_kv_heads;
    // threads past the end still take part in the group shuffles (a group is
    // always inside one wave because G/8 divides 64 and d/8)
    const bool live = tid < n_rows * chunks;
    const int64_t row = live ? tid / chunks : 0;
    append_one<KC, ROLE_K>(a, pl, a.x[0], (int)(row / pl.n_kv_heads), (int)(row % pl.n_kv_heads),
                           (int)(tid % chunks), live);
}

// V plane: a workgroup takes 32 consecutive tokens of one kv-head.  A V-role
// code word holds one channel of eight rows, so storing row by row needs an
// atomic clear and set per nibble (or a byte store per value).  When the 32
// tokens are one whole, aligned block of one sequence (the bulk case: a
// prefill chunk), the workgroup quantizes the 32 rows into an LDS tile and
// writes every word of the block whole, coalesced; otherwise each value goes
// its own way as in the K plane.
constexpr int kVTileStride = 256 + 8;  // bytes per row of the LDS code tile (head_dim <= 256)

template <int VC>
__device__ __forceinline__ void append_v(const AppendArgs &a, int tb, int head) {
    const PlaneView &pl = a.plane[1];
    const int d = pl.head_dim;
    const int chunks = d / 8;
    const int t0 = tb * kBlockRows;
    const int rows = min(kBlockRows, a.n_tokens - t0);
    const int tid = threadIdx.x;
    __shared__ __align__(16) int8_t tile[kBlockRows * kVTileStride];

    // one aligned block of one sequence, every row in range?
    int ok = 1;
    int32_t sq0 = 0;
    int64_t pos0 = 0, head_lin = 0, prow0 = 0;
    if (rows == kBlockRows) {
        sq0 = a.seq_idx[t0];
        pos0 = a.pos[t0];
        if (tid < kBlockRows) ok = a.seq_idx[t0 + tid] == sq0 && a.pos[t0 + tid] == pos0 + tid;
        const int n_seqs = a.pt.table ? a.pt.n_seqs : pl.n_seqs;
        const int64_t cap = a.pt.table ? (int64_t)a.pt.table_stride * a.pt.page_rows : pl.capacity;
        // a page holds whole blocks, so one lookup places all 32 rows
        ok = ok && sq0 >= 0 && sq0 < n_seqs && pos0 >= 0 && pos0 % kBlockRows == 0 &&
             pos0 + kBlockRows <= cap && phys_row(pl, a.pt, sq0, head, pos0, head_lin, prow0);
    } else {
        ok = 0;
    }
    // f16 values are whole 2-byte stores of their own: never the tile
    if (is16(VC)) ok = 0;
    if (!__syncthreads_and(ok)) {
        for (int it = tid; it < ((rows * chunks + 255) / 256) * 256; it += 256)
            append_one<VC, ROLE_V>(a, pl, a.x[1], t0 + it / chunks, head, it % chunks, it < rows * chunks);
        return;
    }

    if constexpr (is16(VC)) return;
    // quantize: codes into the tile [row][channel], scales straight to the block
    const int64_t blk_idx = prow0 / kBlockRows;
    uint8_t *blk = pl.codes + head_lin * pl.head_code_stride + blk_idx * block_code_bytes(VC, d);
    uint16_t *sblk = pl.scales + head_lin * pl.head_scale_stride + blk_idx * block_scales(VC, d);
    constexpr int lanes_per_group = group_size(VC) / 8;
    for (int it = tid; it < kBlockRows * chunks; it += 256) {
        const int r = it / chunks, chunk = it % chunks;
        const float4 *src = reinterpret_cast<const float4 *>(
            a.x[1] + ((int64_t)(t0 + r) * pl.n_kv_heads + head) * d + chunk * 8);
        const float4 v0 = src[0], v1 = src[1];
        const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        int q[8];
        const _Float16 d16 = quantize8<VC>(x, q);
        uint32_t w0 = 0, w1 = 0;
        for (int s = 0; s < 4; ++s) w0 |= (uint32_t)(uint8_t)(int8_t)q[s] << (8 * s);
        for (int s = 0; s < 4; ++s) w1 |= (uint32_t)(uint8_t)(int8_t)q[4 + s] << (8 * s);
        *reinterpret_cast<u2 *>(tile + r * kVTileStride + chunk * 8) = u2{w0, w1};
        if (chunk % lanes_per_group == 0)
            sblk[v_scale_index(VC, d, r, chunk / lanes_per_group)] = __builtin_bit_cast(uint16_t, d16);
    }
    __syncthreads();

    // assemble the block's words in its chunk-major lane order: lane L =
    // c16 + 16 kq owns channel 16 cb + c16 of rows (s/4)*16 + 4 kq + s%4 in
    // slots s = 0..7 (4-bit: slot s in nibble position slot_nibble(s) of one
    // word; 8-bit: slot s in byte s of two words)
    const int LB = v_lane_bytes(VC, d), CW = chunk_width(LB), wpc = CW / 4;
    const int words = kBlockRows * row_bytes(VC, d) / 4;
    for (int w = tid; w < words; w += 256) {
        const int wic = w % wpc, L = (w / wpc) % 64, c = w / wpc / 64;
        const int b = c * CW + wic * 4;  // lane byte
        const int c16 = L & 15, kq = L >> 4;
        uint32_t word = 0;
        if constexpr (is8(VC)) {
            const int ch = 16 * (b / 8) + c16, s0 = b % 8;
            for (int i = 0; i < 4; ++i) {
                const int s = s0 + i, j = (s >> 2) * 16 + 4 * kq + (s & 3);
                word |= (uint32_t)(uint8_t)tile[j * kVTileStride + ch] << (8 * i);
            }
        } else {
            const int ch = 16 * (b / 4) + c16;
            for (int s = 0; s < 8; ++s) {
                const int j = (s >> 2) * 16 + 4 * kq + (s & 3);
                const int q = tile[j * kVTileStride + ch];
                const uint32_t nib = VC == Q4_0 ? (uint32_t)(q + 8) : ((uint32_t)q & 0xFu);
                word |= nib << (4 * slot_nibble(s));
            }
        }
        *reinterpret_cast<uint32_t *>(blk + c * 64 * CW + L * CW + wic * 4) = word;
    }
}

// grid.y = 0: K plane (one thread per 8 channels of a row), 1: V plane (one
// workgroup per 32 tokens and kv-head); one launch appends both.
template <int KC, int VC>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
    if (blockIdx.y == 0) {
        if (a.x[0]) append_k<KC>(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    } else {
        const int H = a.plane[1].n_kv_heads;
        const int tb = (int)(blockIdx.x / H), head = (int)(blockIdx.x % H);
        if (a.x[1] && tb * kBlockRows < a.n_tokens) append_v<VC>(a, tb, head);
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
        if constexpr (is16(CODEC)) {  // the stored binary16 value, exact in fp32
            o[s] = (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t *>(blk + p.byte));
            continue;
        }
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
    if (a.plane[1].head_dim > 256) return hipErrorInvalidValue;  // the V code tile's row
    // K: one thread per 8 channels of a row; V: one workgroup per 32 tokens
    // and kv-head; workgroups past their plane's count return at once
    const int64_t gk = (threads + 255) / 256;
    const int64_t gv = (int64_t)((a.n_tokens + kBlockRows - 1) / kBlockRows) * a.plane[1].n_kv_heads;
    const dim3 block(256), grid((unsigned)(gk > gv ? gk : gv), 2);
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
        case F16 * 3 + F16: append_kernel<F16, F16><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool append_supported(int k_codec, int v_codec) {
    return (k_codec == F16) == (v_codec == F16) && k_codec >= 0 && k_codec <= 3 && v_codec >= 0 && v_codec <= 3;
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
        case F16 * 2 + ROLE_K: dequant_kernel<F16, ROLE_K><<<grid, block, 0, s>>>(a); break;
        case F16 * 2 + ROLE_V: dequant_kernel<F16, ROLE_V><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
