// attn_prefill.hip -- chunked-prefill attention over the block-quantized cache
// on bf16 matrix cores.  gfx950.
//
// What is computed (den_llama.cpp, "Results": prefill with 2048-token
// micro-batches over a q8_0 K / q4_0 V cache; Llaminar, "Graphs and Compute
// Stages": the chunk's rows are appended before attention): for chunk token t
// at absolute position pos0 + t and q-head h,
//   out[t][h] = sum_{j <= pos0+t} softmax_j(scale * q[t][h] . k_hat_j) v_hat_j.
//
// Design:
//  * A "column" is one (token, head) pair of a kv-head's GQA group, ordered
//    token-major.  A workgroup of 8 waves owns 256 consecutive columns (16*NT
//    per wave) of one kv-head, so every K/V tile it dequantizes serves all of
//    them; tiles are 64 rows (two cache blocks).
//  * Per tile, the workgroup dequantizes K and V into LDS as bf16 (code *
//    scale, rounded to nearest even once): K_hat row-major, V_hat transposed
//    [channel][row].  The V-role block layout hands each thread the eight rows
//    of one channel, so the transposed writes are two 8-byte runs.
//  * Each wave computes S^T = K_hat Q^T (A = K_hat rows from LDS, B = its bf16
//    query columns held in registers) and O^T += V_hat^T P^T on
//    v_mfma_f32_16x16x32_bf16.  The S^T accumulator layout is the P^T operand
//    layout, as in the decode kernel.  Online softmax in log2 units with fp32
//    statistics; the running max is raised only when exceeded by more than 8.
//  * Causal mask only on tiles that cross a column's diagonal; rows past the
//    needed range get a zero V so never-written bytes cannot leak NaN.
//  * The two LDS tile buffers alternate, so the dequant of tile k+1 overlaps
//    the products of tile k; tile k+2's codes are loaded into registers and
//    its scales staged in LDS during iteration k, so the dequant never waits
//    for memory.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kTileRows = 64;
constexpr float kPRescaleThreshold = 8.0f;

typedef uint16_t bfbits;

template <int D, int KC, int VC>
struct PCfg {
    static constexpr int KSTEPS = D / 32;
    static constexpr int CB = D / 16;
    static constexpr int NT = D == 256 ? 1 : 2;  // 16-column tiles per wave
    static constexpr int COLS = kPWaves * 16 * NT;
    static constexpr int KG = group_size(KC);
    static constexpr int VG = group_size(VC);
    static constexpr int K_LB = k_lane_bytes(KC, D);
    static constexpr int V_LB = v_lane_bytes(VC, D);
    static constexpr int K_W = chunk_width(K_LB);
    static constexpr int V_W = chunk_width(V_LB);
    static constexpr int K_TILE_BYTES = 16 * row_bytes(KC, D);
    static constexpr int K_BLOCK_BYTES = block_code_bytes(KC, D);
    static constexpr int V_BLOCK_BYTES = block_code_bytes(VC, D);
    static constexpr int K_BLOCK_SCALES = block_scales(KC, D);
    static constexpr int V_BLOCK_SCALES = block_scales(VC, D);
    // dequant work units per 64-row tile (one unit = one lane chunk of W bytes)
    static constexpr int K_UNITS = 2 * 2 * (K_LB / K_W) * 64;
    static constexpr int V_UNITS = 2 * (V_LB / V_W) * 64;
    // LDS tiles (bf16): K_hat [64][KS], V_hat^T [D][VS]; the pads keep the
    // 16-lane groups of the operand reads on distinct banks.  V_hat^T rows are
    // read and written 8 bytes per lane: a row stride of 34 dwords (2 mod 4)
    // measured fastest (a 36-dword stride costs 5 %, 40 dwords 25 %, an
    // unpadded 32 three times the kernel time)
    static constexpr int KS = D + 8;
    static constexpr int VS = kTileRows + 4;
    static constexpr int K_TILE_ELEMS = kTileRows * KS;
    static constexpr int V_TILE_ELEMS = D * VS;
    static constexpr int BUF_ELEMS = K_TILE_ELEMS + V_TILE_ELEMS;
    // dequant units per thread, and a tile's scales (both blocks, K then V)
    static constexpr int UK = (K_UNITS + kPThreads - 1) / kPThreads;
    static constexpr int UV = (V_UNITS + kPThreads - 1) / kPThreads;
    static constexpr int KSC_BYTES = 2 * 2 * K_BLOCK_SCALES;
    static constexpr int VSC_BYTES = 2 * 2 * V_BLOCK_SCALES;
    static constexpr int SC_BYTES = KSC_BYTES + VSC_BYTES;
    static_assert(KSC_BYTES % 16 == 0 && VSC_BYTES % 16 == 0, "scale spans are whole 16-byte pieces");
    static_assert(SC_BYTES / 16 <= kPThreads, "one 16-byte scale piece per thread");
};

__device__ __forceinline__ bfbits to_bf16(float x) {
    return __builtin_bit_cast(bfbits, (__bf16)x);  // round to nearest even
}

// Signed code of the element in nibble position p of a 4-bit word.
template <int CODEC>
__device__ __forceinline__ int nibble_code(uint32_t w, int p) {
    if constexpr (CODEC == Q4_0) return (int)((w >> (4 * p)) & 0xFu) - 8;
    else return ((int)(w << (28 - 4 * p))) >> 28;  // sign-extend the two's complement nibble
}

// Byte offset, within the tile's two K blocks, of K dequant unit u (lane L's
// W-byte chunk c of tile tau of block blk).
template <int D, int KC, int VC>
__device__ __forceinline__ int k_unit_offset(int u) {
    using C = PCfg<D, KC, VC>;
    constexpr int CH = C::K_LB / C::K_W;
    const int L = u & 63, c = (u >> 6) % CH, tau = (u >> 6) / CH % 2, blk = (u >> 6) / CH / 2;
    return blk * C::K_BLOCK_BYTES + tau * C::K_TILE_BYTES + c * 64 * C::K_W + L * C::K_W;
}
template <int D, int KC, int VC>
__device__ __forceinline__ int v_unit_offset(int u) {
    using C = PCfg<D, KC, VC>;
    constexpr int CH = C::V_LB / C::V_W;
    const int L = u & 63, c = (u >> 6) % CH, blk = (u >> 6) / CH;
    return blk * C::V_BLOCK_BYTES + c * 64 * C::V_W + L * C::V_W;
}

// Loads the W bytes at src into words (W = 4, 8 or 16).
template <int W>
__device__ __forceinline__ void load_chunk(uint32_t (&w)[W / 4], const uint8_t *src) {
    if constexpr (W == 16) {
        const u4 v = *reinterpret_cast<const u4 *>(src);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (W == 8) {
        const u2 v = *reinterpret_cast<const u2 *>(src);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(src);
    }
}

// Dequantize K unit u from its code words w into K_hat rows; ksc: the tile's
// K scales (both blocks) in LDS.
template <int D, int KC, int VC>
__device__ __forceinline__ void deq_k_unit(int u, const uint32_t (&w)[PCfg<D, KC, VC>::K_W / 4],
                                           const uint16_t *ksc0, bfbits *khat) {
    using C = PCfg<D, KC, VC>;
    constexpr int CH = C::K_LB / C::K_W;
    const int L = u & 63;
    const int c = (u >> 6) % CH;
    const int tau = (u >> 6) / CH % 2;
    const int blk = (u >> 6) / CH / 2;
    const uint16_t *ksc = ksc0 + blk * C::K_BLOCK_SCALES;
    const int i = L & 15, kq = L >> 4;
    const int j = tau * 16 + i;        // row in block
    const int row = blk * 32 + j;      // row in tile
    constexpr int STEPS = is8(KC) ? C::K_W / 8 : C::K_W / 4;  // k-steps in this chunk
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int t = c * STEPS + st;
        const int g = (32 * t) / C::KG;
        const float dq = (float)__builtin_bit_cast(_Float16, ksc[k_scale_index(KC, D, j, g)]);
        bfbits o[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            int code;
            if constexpr (is8(KC)) code = (int)(int8_t)((w[2 * st + (s >> 2)] >> (8 * (s & 3))) & 0xFFu);
            else code = nibble_code<KC>(w[st], slot_nibble(s));
            o[s] = to_bf16((float)code * dq);
        }
        u4 pk;
        pk.x = o[0] | ((uint32_t)o[1] << 16);
        pk.y = o[2] | ((uint32_t)o[3] << 16);
        pk.z = o[4] | ((uint32_t)o[5] << 16);
        pk.w = o[6] | ((uint32_t)o[7] << 16);
        *reinterpret_cast<u4 *>(khat + row * C::KS + 32 * t + 8 * kq) = pk;
    }
}

// Dequantize V unit u from its code words into V_hat^T [channel][row]; vsc0:
// the tile's V scales (both blocks) in LDS; rows at or past `vrows`
// (tile-relative) are written as zero.
template <int D, int KC, int VC>
__device__ __forceinline__ void deq_v_unit(int u, const uint32_t (&w)[PCfg<D, KC, VC>::V_W / 4],
                                           const uint16_t *vsc0, bfbits *vhat, int vrows) {
    using C = PCfg<D, KC, VC>;
    constexpr int CH = C::V_LB / C::V_W;
    const int L = u & 63;
    const int c = (u >> 6) % CH;
    const int blk = (u >> 6) / CH;
    const uint16_t *vsc = vsc0 + blk * C::V_BLOCK_SCALES;
    const int c16 = L & 15, kq = L >> 4;
    constexpr int CBS = is8(VC) ? C::V_W / 8 : C::V_W / 4;  // channel blocks in this chunk
#pragma unroll
    for (int k = 0; k < CBS; ++k) {
        const int cb = c * CBS + k;
        const int ch = 16 * cb + c16;
        const int g = (16 * cb) / C::VG;
        bfbits o[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int j = (s >> 2) * 16 + 4 * kq + (s & 3);  // row in block
            const float dq = (float)__builtin_bit_cast(_Float16, vsc[v_scale_index(VC, D, j, g)]);
            int code;
            if constexpr (is8(VC)) code = (int)(int8_t)((w[2 * k + (s >> 2)] >> (8 * (s & 3))) & 0xFFu);
            else code = nibble_code<VC>(w[k], slot_nibble(s));
            o[s] = blk * 32 + j < vrows ? to_bf16((float)code * dq) : (bfbits)0;
        }
        // slots 0..3 are rows 4kq..4kq+3, slots 4..7 rows 16+4kq..16+4kq+3
        bfbits *dst = vhat + ch * C::VS + blk * 32 + 4 * kq;
        *reinterpret_cast<u2 *>(dst) = u2{o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16)};
        *reinterpret_cast<u2 *>(dst + 16) = u2{o[4] | ((uint32_t)o[5] << 16), o[6] | ((uint32_t)o[7] << 16)};
    }
}

template <int D, int KC, int VC>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a) {
    using C = PCfg<D, KC, VC>;
    extern __shared__ __align__(16) unsigned char smem[];
    bfbits *lds = reinterpret_cast<bfbits *>(smem);

    const int G = a.gqa;
    const int kvh = blockIdx.y;
    const int ncols = a.n_tokens * G;
    const int col0 = blockIdx.x * C::COLS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h16 = lane & 15, q4 = lane >> 4;

    // rows this workgroup needs: [0, pos0 + last token + 1)
    const int last_col = min(col0 + C::COLS, ncols) - 1;
    const int64_t nrows = a.pos0 + last_col / G + 1;
    const int ntiles = (int)((nrows + kTileRows - 1) / kTileRows);

    // ---- this wave's bf16 query columns (B operand of S^T), zero past the end
    bf8 qop[C::NT][C::KSTEPS];
    int diag[C::NT];  // absolute position of this lane's column (its last visible row)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        const int col = col0 + (wave * C::NT + nt) * 16 + h16;
        const bool ok = col < ncols;
        const int t = ok ? col / G : 0, hh = ok ? col % G : 0;
        diag[nt] = ok ? (int)(a.pos0 + t) : -1;
        const uint16_t *qp = a.q + ((int64_t)t * a.n_q_heads + (int64_t)kvh * G + hh) * D;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            u4 v = ok ? *reinterpret_cast<const u4 *>(qp + 32 * ks + 8 * q4) : u4{0u, 0u, 0u, 0u};
            qop[nt][ks] = __builtin_bit_cast(bf8, v);
        }
    }

    const int64_t head_lin = (int64_t)a.seq * a.k.n_kv_heads + kvh;
    const uint8_t *kcodes = a.k.codes + head_lin * a.k.head_code_stride;
    const uint8_t *vcodes = a.v.codes + head_lin * a.v.head_code_stride;
    const uint16_t *kscales = a.k.scales + head_lin * a.k.head_scale_stride;
    const uint16_t *vscales = a.v.scales + head_lin * a.v.head_scale_stride;
    const int64_t nblocks_plane = a.k.capacity / kBlockRows;

    // The tile pipeline: a tile's codes are loaded into registers and its
    // scales staged in LDS one iteration before it is dequantized, which is
    // one iteration before its products, so neither the global loads nor the
    // dequant wait in line with the matrix products.
    uint32_t rk[C::UK][C::K_W / 4], rv[C::UV][C::V_W / 4];
    u4 rsc = u4{0u, 0u, 0u, 0u};
    uint16_t *sc_lds = reinterpret_cast<uint16_t *>(lds + 2 * C::BUF_ELEMS);  // [2][SC_BYTES / 2]
    auto load_tile = [&](int tile) {
        const int64_t b0 = (int64_t)tile * 2;  // first block of the tile
        const bool two = b0 + 1 < nblocks_plane;  // the second block exists
        const uint8_t *kb = kcodes + b0 * C::K_BLOCK_BYTES;
        const uint8_t *vb = vcodes + b0 * C::V_BLOCK_BYTES;
#pragma unroll
        for (int i = 0; i < C::UK; ++i) {
            const int u = tid + i * kPThreads;
            if (u < C::K_UNITS && (two || u < C::K_UNITS / 2)) load_chunk<C::K_W>(rk[i], kb + k_unit_offset<D, KC, VC>(u));
        }
#pragma unroll
        for (int i = 0; i < C::UV; ++i) {
            const int u = tid + i * kPThreads;
            if (u < C::V_UNITS && (two || u < C::V_UNITS / 2)) load_chunk<C::V_W>(rv[i], vb + v_unit_offset<D, KC, VC>(u));
        }
        // the tile's scales, 16 bytes per thread: K (both blocks) then V
        const int o = tid * 16;
        if (o < C::KSC_BYTES) {
            if (two || o < C::KSC_BYTES / 2)
                rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(kscales + b0 * C::K_BLOCK_SCALES) + o);
        } else if (o < C::SC_BYTES) {
            const int ov = o - C::KSC_BYTES;
            if (two || ov < C::VSC_BYTES / 2)
                rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(vscales + b0 * C::V_BLOCK_SCALES) + ov);
        }
    };
    auto stage_scales = [&](int tile) {
        if (tid * 16 < C::SC_BYTES)
            *reinterpret_cast<u4 *>(reinterpret_cast<uint8_t *>(sc_lds + (tile & 1) * (C::SC_BYTES / 2)) + tid * 16) = rsc;
    };
    // dequantizes the tile whose codes are in rk/rv and whose scales are staged
    auto dequant_tile = [&](int tile, bfbits *buf) {
        const int64_t b0 = (int64_t)tile * 2;
        const int vrows = (int)min((int64_t)kTileRows, nrows - (int64_t)tile * kTileRows);
        const bool two = b0 + 1 < nblocks_plane;
        const uint16_t *ksc = sc_lds + (tile & 1) * (C::SC_BYTES / 2);
        const uint16_t *vsc = ksc + C::KSC_BYTES / 2;
        bfbits *khat = buf;
        bfbits *vhat = buf + C::K_TILE_ELEMS;
#pragma unroll
        for (int i = 0; i < C::UK; ++i) {
            const int u = tid + i * kPThreads;
            if (u >= C::K_UNITS || (!two && u >= C::K_UNITS / 2)) continue;  // block 1 absent: rows unused
            deq_k_unit<D, KC, VC>(u, rk[i], ksc, khat);
        }
#pragma unroll
        for (int i = 0; i < C::UV; ++i) {
            const int u = tid + i * kPThreads;
            if (u >= C::V_UNITS) continue;
            if (!two && u >= C::V_UNITS / 2) {
                // absent block: zero its V columns so masked products stay 0
                const int L = u & 63, c16 = L & 15, kq = L >> 4;
                constexpr int CH = C::V_LB / C::V_W;
                constexpr int CBS = is8(VC) ? C::V_W / 8 : C::V_W / 4;
                const int c = (u >> 6) % CH;
#pragma unroll
                for (int k = 0; k < CBS; ++k) {
                    bfbits *dst = vhat + (16 * (c * CBS + k) + c16) * C::VS + 32 + 4 * kq;
                    *reinterpret_cast<u2 *>(dst) = u2{0u, 0u};
                    *reinterpret_cast<u2 *>(dst + 16) = u2{0u, 0u};
                }
                continue;
            }
            deq_v_unit<D, KC, VC>(u, rv[i], vsc, vhat, vrows);
        }
    };

    f4 O[C::NT][C::CB];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) O[nt][cb] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run[C::NT], l_run[C::NT];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.0f;
    }
    // smallest and largest diagonal over this wave's valid columns
    int wave_min_diag;
    {
        // lanes past the end have diag -1; take the minimum over valid ones
        int v = diag[0] < 0 ? INT32_MAX : diag[0];
#pragma unroll
        for (int nt = 1; nt < C::NT; ++nt) v = min(v, diag[nt] < 0 ? INT32_MAX : diag[nt]);
        for (int m = 1; m < 64; m <<= 1) v = min(v, __shfl_xor(v, m, 64));
        wave_min_diag = v;
    }
    int wave_max_diag;
    {
        int v = diag[0];
#pragma unroll
        for (int nt = 1; nt < C::NT; ++nt) v = max(v, diag[nt]);
        for (int m = 1; m < 64; m <<= 1) v = max(v, __shfl_xor(v, m, 64));
        wave_max_diag = v;  // -1 when the wave has no valid column
    }

    // prologue: tile 0 dequantized, tile 1 loaded and its scales staged
    load_tile(0);
    stage_scales(0);
    __syncthreads();
    dequant_tile(0, lds);
    if (1 < ntiles) {
        load_tile(1);
        stage_scales(1);
    }
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
        bfbits *cur = lds + (tile & 1) * C::BUF_ELEMS;
        if (tile + 1 < ntiles) dequant_tile(tile + 1, lds + ((tile + 1) & 1) * C::BUF_ELEMS);
        if (tile + 2 < ntiles) load_tile(tile + 2);
        const int row0 = tile * kTileRows;
        if (row0 <= wave_max_diag) {  // some column of this wave sees rows of this tile
            const bfbits *khat = cur;
            const bfbits *vhat = cur + C::K_TILE_ELEMS;
            // ---- S^T: 4 row tiles x NT column tiles
            f4 S[C::NT][4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                bf8 kop[C::KSTEPS];
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks)
                    kop[ks] = *reinterpret_cast<const bf8 *>(khat + (16 * mt + h16) * C::KS + 32 * ks + 8 * q4);
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) {
                    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < C::KSTEPS; ++ks) acc = mfma16x16x32_bf16(kop[ks], qop[nt][ks], acc);
                    S[nt][mt] = acc * a.scale_log2;
                }
            }
            const bool diag_tile = row0 + kTileRows - 1 > wave_min_diag;
            // P^T operands: k-step ks covers row tiles 2ks, 2ks+1
            bf8 P[C::NT][2];
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) {
                if (diag_tile) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (row0 + 16 * mt + 4 * q4 + r > diag[nt]) S[nt][mt][r] = -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[nt][mt][r]);
                mx = fmaxf(mx, shfl_xor(mx, 16));
                mx = fmaxf(mx, shfl_xor(mx, 32));
                // a column with every row of this tile masked keeps its state
                const bool raise = mx > m_run[nt] + kPRescaleThreshold;
                if (__any(raise)) {
                    const float m_new = raise ? mx : m_run[nt];
                    const float alpha = raise ? fast_exp2(m_run[nt] - m_new) : 1.0f;
                    l_run[nt] *= alpha;
#pragma unroll
                    for (int cb = 0; cb < C::CB; ++cb) O[nt][cb] *= alpha;
                    m_run[nt] = m_new;
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p = fast_exp2(S[nt][mt][r] - m_run[nt]);  // 0 when masked
                        l_run[nt] += p;
                        P[nt][mt >> 1][4 * (mt & 1) + r] = (__bf16)p;
                    }
            }
            // ---- O^T += V_hat^T P^T; each V_hat operand read serves every
            // column tile of the wave
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bfbits *vp = vhat + (16 * cb + h16) * C::VS + 32 * ks + 4 * q4;
                    const u2 lo = *reinterpret_cast<const u2 *>(vp);
                    const u2 hi = *reinterpret_cast<const u2 *>(vp + 16);
                    const bf8 vop = __builtin_bit_cast(bf8, u4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int nt = 0; nt < C::NT; ++nt) O[nt][cb] = mfma16x16x32_bf16(vop, P[nt][ks], O[nt][cb]);
                }
            }
        }
        // tile + 2's scales go where tile's were (read by its dequant, one
        // iteration ago)
        if (tile + 2 < ntiles) stage_scales(tile + 2);
        __syncthreads();  // next tile's dequant and staging done; this tile's reads done
    }

    // ---- normalize and store: lane (column h16, q4) holds channels 16cb+4q4..+3
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        float L = l_run[nt];
        L += shfl_xor(L, 16);
        L += shfl_xor(L, 32);
        if (diag[nt] < 0) continue;
        const int col = col0 + (wave * C::NT + nt) * 16 + h16;
        const int t = col / G, hh = col % G;
        float *dst = a.out + ((int64_t)t * a.n_q_heads + (int64_t)kvh * G + hh) * D;
        const float inv = 1.0f / L;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
            *reinterpret_cast<f4 *>(dst + 16 * cb + 4 * q4) = O[nt][cb] * inv;
    }
}

template <int D, int KC, int VC>
hipError_t launch_ptyped(const PrefillArgs &a, hipStream_t s) {
    using C = PCfg<D, KC, VC>;
    const size_t lds = 2 * (size_t)C::BUF_ELEMS * sizeof(bfbits) + 2 * (size_t)C::SC_BYTES;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_kernel<D, KC, VC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int ncols = a.n_tokens * a.gqa;
    const dim3 grid((unsigned)((ncols + C::COLS - 1) / C::COLS), (unsigned)a.k.n_kv_heads);
    prefill_kernel<D, KC, VC><<<grid, dim3(kPThreads), lds, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_pd(const PrefillArgs &a, hipStream_t s) {
    switch (a.k.codec * 3 + a.v.codec) {
        case Q8_0 * 3 + Q8_0: return launch_ptyped<D, Q8_0, Q8_0>(a, s);
        case Q8_0 * 3 + Q4_0: return launch_ptyped<D, Q8_0, Q4_0>(a, s);
        case Q8_0 * 3 + Q4_G64: return launch_ptyped<D, Q8_0, Q4_G64>(a, s);
        case Q4_0 * 3 + Q8_0: return launch_ptyped<D, Q4_0, Q8_0>(a, s);
        case Q4_0 * 3 + Q4_0: return launch_ptyped<D, Q4_0, Q4_0>(a, s);
        case Q4_0 * 3 + Q4_G64: return launch_ptyped<D, Q4_0, Q4_G64>(a, s);
        case Q4_G64 * 3 + Q8_0: return launch_ptyped<D, Q4_G64, Q8_0>(a, s);
        case Q4_G64 * 3 + Q4_0: return launch_ptyped<D, Q4_G64, Q4_0>(a, s);
        case Q4_G64 * 3 + Q4_G64: return launch_ptyped<D, Q4_G64, Q4_G64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool prefill_supported(int k_codec, int v_codec, int head_dim) {
    return k_codec >= 0 && k_codec <= 2 && v_codec >= 0 && v_codec <= 2 &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    switch (a.k.head_dim) {
        case 64: return launch_pd<64>(a, s);
        case 128: return launch_pd<128>(a, s);
        case 256: return launch_pd<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
