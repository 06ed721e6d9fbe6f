// attn_prefill.hip -- chunked-prefill attention over the block-quantized cache
// on binary16 matrix cores.  gfx950.
//
// What is computed (den_llama.cpp, "Results": prefill with 2048-token
// micro-batches over a q8_0 K / q4_0 V cache; Llaminar, "Graphs and Compute
// Stages": the chunk's rows are appended before attention): for chunk token t
// at absolute position pos0 + t and q-head h,
//   out[t][h] = sum_{j <= pos0+t} softmax_j(scale * q[t][h] . k_hat_j) v_hat_j.
//
// Design:
//  * A "column" is one (token, head) pair of a kv-head's GQA group, ordered
//    token-major.  A workgroup owns consecutive columns of one kv-head (16*NT
//    per wave: 8 waves of 32 at head_dim 128, 12 of 16 at 256, 16 of 16 at
//    64), so every K/V tile it dequantizes serves all of them; tiles are 64
//    rows (two cache blocks).
//  * Per tile, the workgroup dequantizes K and V into LDS as binary16 (code *
//    scale, rounded to nearest even once): K_hat row-major, V_hat transposed
//    [channel][row].  Codes become exact binary16 pairs by bit operations
//    (1024 + n), so a pair of values costs one packed subtract and one packed
//    multiply; the work is cut into units so that every thread dequantizes
//    the same number of values.  The V-role block layout hands each thread
//    the eight rows of one channel, so the transposed writes are two 8-byte
//    runs.
//  * The bf16 query is widened and scaled by a power of two per (token,
//    head) column so that its largest value lies in [1, 2), then rounded to
//    binary16 (exact for every value within 2^-14 of that maximum); the power
//    of two is folded into the column's score scale.  The softmax scale's
//    sign goes into the query as well, so the column's factor is positive:
//    the maximum is taken over the raw scores, and the factor multiplies a
//    score inside the FMA that subtracts the running maximum before exp2.
//  * The 8 XCDs each have their own L2 and receive workgroups round-robin;
//    the column groups of one kv-head are placed on one XCD, so the K/V rows
//    they all sweep come from HBM about once per kv-head.
//  * Each wave computes S^T = K_hat Q^T (A = K_hat rows from LDS, B = its
//    query columns held in registers) and O^T += V_hat^T P^T on
//    v_mfma_f32_16x16x32_f16.  The S^T accumulator layout is the P^T operand
//    layout, as in the decode kernel.  Online softmax in log2 units with fp32
//    statistics; the running max is raised only when exceeded by more than 8
//    (so probabilities stay <= 256 in binary16).
//  * Causal mask only on tiles that cross a column's diagonal; rows past the
//    needed range get a zero V so never-written bytes cannot leak NaN.
//  * The two LDS tile buffers alternate, so the dequant of tile k+1 overlaps
//    the products of tile k; tile k+2's codes are loaded into registers and
//    its scales staged in LDS during iteration k, so the dequant never waits
//    for memory.
#include <cfloat>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

// waves per workgroup: 8 of 32 columns at head_dim 128; 12 of 16 columns at
// head_dim 256 (so that a 2048-token chunk of 6-head groups over 4 kv-heads is
// 256 workgroups, one round on the 256 compute units, instead of 384); 16 of
// 16 columns at head_dim 64 (four waves per SIMD fit in 128 VGPRs there)
constexpr int prefill_waves(int d) { return d == 256 ? 12 : (d == 64 ? 16 : 8); }
constexpr int kTileRows = 64;
constexpr float kPRescaleThreshold = 8.0f;

typedef uint16_t f16bits;

constexpr int clamp_width(int w, int lo, int hi) { return w < lo ? lo : (w > hi ? hi : w); }

// A wait for every vector-memory load of this wave, where all of them have
// landed anyway (the dequant has just consumed the previous tile's codes).
// It is there for the compiler: a code register is loaded and dequantized
// under conditions it cannot match up (units past the tile's count), so it
// treats each one as possibly still in flight from an earlier iteration, and
// before reloading it would wait for every load issued so far -- including
// the ones of this tile just sent -- which lines up the tile's loads one
// memory round trip after another.  After this wait nothing is in flight and
// the loads go out together.  (A builtin, not inline assembly: the compiler's
// wait bookkeeping sees it.)  Used where every wave runs the same iteration
// (head_dim 256, where this happened: 2.34 -> 2.24 ms for q8_0 / q4_0); with
// the two wave groups the loads already go out together.
__device__ __forceinline__ void loads_landed() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left at their maxima
}

// Scheduling directive for a block of NR LDS operand reads feeding NM matrix
// products: LEAD reads first, then each read follows NM / NR products, so
// LEAD reads stay in flight ahead of the products that use them (left to
// itself the scheduler waits on each read right after issuing it).  Four
// reads ahead measured fastest with 8 waves (2, 3, 5, 8 and 12 tried; 6 spills
// at head_dim 128) and with the 16 waves of head_dim 64 (6 and 8 no faster);
// with the 12 waves of head_dim 256 (168 VGPRs each) two measured fastest (one
// and three slower, the latter by 20 % for q8_0 / q4_0).
template <int D>
constexpr int read_lead() { return D == 256 ? 2 : 4; }
template <int NR, int NM, int LEAD_>
__device__ __forceinline__ void reads_ahead_of_products() {
    constexpr int LEAD = LEAD_ < NR ? LEAD_ : NR - 1;
    static_assert(LEAD > 0 && NM % NR == 0, "whole products per read");
    __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < NR - LEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);  // matrix products
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM / NR * LEAD, 0);
}

template <int D, int KC, int VC, bool PAGED = false>
struct PCfg {
    static constexpr int KSTEPS = D / 32;
    static constexpr int CB = D / 16;
    static constexpr int NT = D == 128 ? 2 : 1;  // 16-column tiles per wave
    static constexpr int WAVES = prefill_waves(D);
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int COLS = WAVES * 16 * NT;
    static constexpr int KG = group_size(KC);
    static constexpr int VG = group_size(VC);
    static constexpr int VNG = D / VG;
    static constexpr int K_LB = k_lane_bytes(KC, D);
    static constexpr int V_LB = v_lane_bytes(VC, D);
    // the cache's chunk widths, and the dequant unit widths: a unit is UW
    // bytes of one lane's chunk, sized so that a 64-row tile has one unit per
    // thread where the codec allows (a unit holds at least one k-step /
    // channel block)
    static constexpr int K_CW = chunk_width(K_LB);
    static constexpr int V_CW = chunk_width(V_LB);
    static constexpr int K_BPS = is8(KC) ? 8 : 4;  // code bytes per k-step per lane
    static constexpr int V_BPC = is8(VC) ? 8 : 4;  // code bytes per channel block per lane
    static constexpr int K_UW = clamp_width(K_LB / 2, K_BPS, K_CW);
    static constexpr int V_UW = clamp_width(V_LB / 4, V_BPC, V_CW);
    static constexpr int K_TILE_BYTES = 16 * row_bytes(KC, D);
    static constexpr int K_BLOCK_BYTES = block_code_bytes(KC, D);
    static constexpr int V_BLOCK_BYTES = block_code_bytes(VC, D);
    static constexpr int K_BLOCK_SCALES = block_scales(KC, D);
    static constexpr int V_BLOCK_SCALES = block_scales(VC, D);
    // dequant units per 64-row tile
    static constexpr int K_UNITS = 2 * 2 * (K_LB / K_UW) * 64;
    static constexpr int V_UNITS = 2 * (V_LB / V_UW) * 64;
    // LDS tiles (binary16): K_hat [64][KS], V_hat^T [D][VS]; the pads keep the
    // 16-lane groups of the operand reads on distinct banks.  V_hat^T rows are
    // read and written 8 bytes per lane: a row stride of 34 dwords (2 mod 4)
    // measured fastest (a 36-dword stride costs 5 %, 40 dwords 25 %, an
    // unpadded 32 three times the kernel time)
    static constexpr int KS = D + 8;
    static constexpr int VS = kTileRows + 4;
    static constexpr int K_TILE_ELEMS = kTileRows * KS;
    static constexpr int V_TILE_ELEMS = D * VS;
    static constexpr int KSC_BYTES_ = 2 * 2 * K_BLOCK_SCALES;
    static constexpr int SC_BYTES_ = KSC_BYTES_ + 2 * 2 * V_BLOCK_SCALES;
    // Two K_hat buffers; three V_hat buffers where LDS allows, so that a
    // tile's V_hat outlives the next tile's K_hat (the two wave groups below
    // run half a tile apart), else two
    static constexpr int PAGE_LDS = PAGED ? 4 * kPrefillMaxPages : 0;  // paged: the sequence's page numbers
    static constexpr int NVB =
        (2 * K_TILE_ELEMS + 3 * V_TILE_ELEMS) * 2 + 2 * SC_BYTES_ + PAGE_LDS <= 160 * 1024 ? 3 : 2;
    static constexpr bool PINGPONG = NVB == 3;
    static constexpr int OFF_V = 2 * K_TILE_ELEMS;               // elements
    static constexpr int OFF_SC = OFF_V + NVB * V_TILE_ELEMS;    // elements
    static constexpr int OFF_PAGES = OFF_SC * 2 + 2 * SC_BYTES_;  // bytes
    static constexpr int LDS_BYTES = OFF_PAGES + PAGE_LDS;
    static_assert(LDS_BYTES <= 160 * 1024, "the tiles fit in LDS");
    // dequant units per thread, and a tile's scales (both blocks, K then V)
    static constexpr int UK = (K_UNITS + THREADS - 1) / THREADS;
    static constexpr int UV = (V_UNITS + THREADS - 1) / THREADS;
    static constexpr int KSC_BYTES = 2 * 2 * K_BLOCK_SCALES;
    static constexpr int VSC_BYTES = 2 * 2 * V_BLOCK_SCALES;
    static constexpr int SC_BYTES = KSC_BYTES + VSC_BYTES;
    static_assert(KSC_BYTES % 16 == 0 && VSC_BYTES % 16 == 0, "scale spans are whole 16-byte pieces");
    static_assert(SC_BYTES / 16 <= THREADS, "one 16-byte scale piece per thread");
    static_assert(K_UW % K_BPS == 0 && V_UW % V_BPC == 0, "units hold whole k-steps / channel blocks");
};

// Unit u of a tile's K codes: lane L, chunk c, sub-unit `sub` of tile tau of
// block blk.
struct KUnit {
    int L, sub, c, tau, blk;
};
template <int D, int KC, int VC>
__device__ __forceinline__ KUnit k_unit(int u) {
    using C = PCfg<D, KC, VC>;
    constexpr int SUB = C::K_CW / C::K_UW, CH = C::K_LB / C::K_CW;
    const int x = u >> 6;
    return KUnit{u & 63, x % SUB, x / SUB % CH, x / SUB / CH % 2, x / SUB / CH / 2};
}
// Byte offset of K unit u within the tile's two K blocks.
template <int D, int KC, int VC>
__device__ __forceinline__ int k_unit_offset(int u) {
    using C = PCfg<D, KC, VC>;
    const KUnit k = k_unit<D, KC, VC>(u);
    return k.blk * C::K_BLOCK_BYTES + k.tau * C::K_TILE_BYTES + k.c * 64 * C::K_CW + k.L * C::K_CW + k.sub * C::K_UW;
}
struct VUnit {
    int L, sub, c, blk;
};
template <int D, int KC, int VC>
__device__ __forceinline__ VUnit v_unit(int u) {
    using C = PCfg<D, KC, VC>;
    constexpr int SUB = C::V_CW / C::V_UW, CH = C::V_LB / C::V_CW;
    const int x = u >> 6;
    return VUnit{u & 63, x % SUB, x / SUB % CH, x / SUB / CH};
}
template <int D, int KC, int VC>
__device__ __forceinline__ int v_unit_offset(int u) {
    using C = PCfg<D, KC, VC>;
    const VUnit v = v_unit<D, KC, VC>(u);
    return v.blk * C::V_BLOCK_BYTES + v.c * 64 * C::V_CW + v.L * C::V_CW + v.sub * C::V_UW;
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

// Dequantize K unit u from its code words w into K_hat rows; ksc0: the tile's
// K scales (both blocks) in LDS.  Every slot of a k-step shares one scale.
template <int D, int KC, int VC>
__device__ __forceinline__ void deq_k_unit(int u, const uint32_t (&w)[PCfg<D, KC, VC>::K_UW / 4],
                                           const uint16_t *ksc0, f16bits *khat) {
    using C = PCfg<D, KC, VC>;
    constexpr int STEPS = C::K_UW / C::K_BPS;  // k-steps in this unit
    const KUnit k = k_unit<D, KC, VC>(u);
    const uint16_t *ksc = ksc0 + k.blk * C::K_BLOCK_SCALES;
    const int i = k.L & 15, kq = k.L >> 4;
    const int j = k.tau * 16 + i;      // row in block
    const int row = k.blk * 32 + j;    // row in tile
    const int t0 = (k.c * C::K_CW + k.sub * C::K_UW) / C::K_BPS;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int t = t0 + st;
        const int g = (32 * t) / C::KG;
        const _Float16 dq = __builtin_bit_cast(_Float16, ksc[k_scale_index(KC, D, j, g)]);
        const h2 dq4[4] = {h2{dq, dq}, h2{dq, dq}, h2{dq, dq}, h2{dq, dq}};
        const h8 x = v_operand<KC>(&w[is8(KC) ? 2 * st : st], reinterpret_cast<const h2_alias *>(dq4));
        *reinterpret_cast<u4 *>(khat + row * C::KS + 32 * t + 8 * kq) = __builtin_bit_cast(u4, x);
    }
}

// Dequantize V unit u from its code words into V_hat^T [channel][row]; vsc0:
// the tile's V scales (both blocks) in LDS.  With `tail`, rows at or past
// `vrows` (tile-relative) get a zero scale, so bytes that were never written
// cannot turn into NaN.
template <int D, int KC, int VC>
__device__ __forceinline__ void deq_v_unit(int u, const uint32_t (&w)[PCfg<D, KC, VC>::V_UW / 4],
                                           const uint16_t *vsc0, f16bits *vhat, bool tail, int vrows) {
    using C = PCfg<D, KC, VC>;
    constexpr int CBS = C::V_UW / C::V_BPC;  // channel blocks in this unit
    const VUnit v = v_unit<D, KC, VC>(u);
    const int c16 = v.L & 15, kq = v.L >> 4;
    const int cb0 = (v.c * C::V_CW + v.sub * C::V_UW) / C::V_BPC;
    // this lane's scale words: [group][pair m] holds slots (2m, 2m+1), i.e.
    // rows (m/2)*16 + 4kq + 2(m%2) + {0, 1} of the block
    const uint32_t *vsw = reinterpret_cast<const uint32_t *>(vsc0 + v.blk * C::V_BLOCK_SCALES + kq * 8 * C::VNG);
#pragma unroll
    for (int k = 0; k < CBS; ++k) {
        const int cb = cb0 + k;
        const int ch = 16 * cb + c16;
        const int g = (16 * cb) / C::VG;
        uint32_t s4[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) s4[m] = vsw[g * 4 + m];
        if (tail) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j0 = v.blk * 32 + (m >> 1) * 16 + 4 * kq + 2 * (m & 1);
                if (j0 >= vrows) s4[m] &= 0xFFFF0000u;
                if (j0 + 1 >= vrows) s4[m] &= 0x0000FFFFu;
            }
        }
        const h8 x = v_operand<VC>(&w[is8(VC) ? 2 * k : k], reinterpret_cast<const h2_alias *>(s4));
        const u4 b = __builtin_bit_cast(u4, x);
        // slots 0..3 are rows 4kq..4kq+3, slots 4..7 rows 16+4kq..16+4kq+3
        f16bits *dst = vhat + ch * C::VS + v.blk * 32 + 4 * kq;
        *reinterpret_cast<u2 *>(dst) = u2{b.x, b.y};
        *reinterpret_cast<u2 *>(dst + 16) = u2{b.z, b.w};
    }
}

// PAGED: the planes are a page pool addressed through a.pt (else contiguous).
template <int D, int KC, int VC, bool PAGED>
__global__ __launch_bounds__(64 * prefill_waves(D), 1) void prefill_kernel(PrefillArgs a) {
    using C = PCfg<D, KC, VC, PAGED>;
    extern __shared__ __align__(16) unsigned char smem[];
    f16bits *lds = reinterpret_cast<f16bits *>(smem);

    const int G = a.gqa;
    const int ncols = a.n_tokens * G;
    // Workgroups are dealt to the 8 XCDs, each with its own L2, round-robin
    // by id.  Every column group of a kv-head sweeps the same K/V rows in the
    // same order, so where the count allows, the groups of one kv-head share
    // an XCD: workgroup L takes entry (L % 8) * (n / 8) + L / 8 of the
    // kv-head-major list of (kv-head, column group) pairs, and its rows come
    // from that XCD's L2 after the first group has read them.
    const int ncg = (ncols + C::COLS - 1) / C::COLS;
    const int nwg = (int)gridDim.x, L = (int)blockIdx.x;
    const int pair = nwg % 8 == 0 ? (L % 8) * (nwg / 8) + L / 8 : L;
    const int kvh = pair / ncg;
    const int col0 = (pair % ncg) * C::COLS;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h16 = lane & 15, q4 = lane >> 4;

    // rows this workgroup needs: [0, pos0 + last token + 1)
    const int last_col = min(col0 + C::COLS, ncols) - 1;
    const int64_t nrows = a.pos0 + last_col / G + 1;
    const int ntiles = (int)((nrows + kTileRows - 1) / kTileRows);

    // ---- this wave's query columns (B operand of S^T), zero past the end:
    // bf16 widened exactly, scaled by 2^-e so the column's largest value lies
    // in [1, 2), rounded to binary16; 2^e goes into the column's score scale
    h8 qop[C::NT][C::KSTEPS];
    int diag[C::NT];       // absolute position of this lane's column (its last visible row)
    float cscale[C::NT];   // score scale of this lane's column (log2 units)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        const int col = col0 + (wave * C::NT + nt) * 16 + h16;
        const bool ok = col < ncols;
        const int t = ok ? col / G : 0, hh = ok ? col % G : 0;
        diag[nt] = ok ? (int)(a.pos0 + t) : -1;
        const uint16_t *qp = a.q + ((int64_t)t * a.n_q_heads + (int64_t)kvh * G + hh) * D;
        u4 raw[C::KSTEPS];
        float mx = 0.0f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            raw[ks] = ok ? *reinterpret_cast<const u4 *>(qp + 32 * ks + 8 * q4) : u4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const uint32_t wd = raw[ks][s2 >> 1];
                mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, (s2 & 1) ? (wd & 0xFFFF0000u) : (wd << 16))));
            }
        }
        mx = quad_max(mx);
        const int e = mx > 0.0f ? ilogbf(mx) : 0;
        // the scale's sign goes into the operand, so the column's factor is
        // positive (at least FLT_MIN: a zero scale still weighs every visible
        // row alike) and the largest raw score gives the largest scaled one
        cscale[nt] = fmaxf(ldexpf(fabsf(a.scale_log2), e), FLT_MIN);
        const bool neg = a.scale_log2 < 0.0f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const uint32_t wd = raw[ks][s2 >> 1];
                const float x = __builtin_bit_cast(float, (s2 & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                qop[nt][ks][s2] = (_Float16)ldexpf(neg ? -x : x, -e);
            }
    }

    const int64_t head_lin = (int64_t)a.seq * a.k.n_kv_heads + kvh;
    const uint8_t *kcodes = a.k.codes + head_lin * a.k.head_code_stride;
    const uint8_t *vcodes = a.v.codes + head_lin * a.v.head_code_stride;
    const uint16_t *kscales = a.k.scales + head_lin * a.k.head_scale_stride;
    const uint16_t *vscales = a.v.scales + head_lin * a.v.head_scale_stride;
    // blocks of the sequence: the capacity of its plane, or of its table
    const int64_t nblocks_plane =
        PAGED ? (int64_t)a.pt.table_stride * (a.pt.page_rows / kBlockRows) : a.k.capacity / kBlockRows;
    // paged: the sequence's page numbers, for every block this workgroup
    // reads, copied to LDS once (read back before every tile load)
    const int32_t *page_lds = reinterpret_cast<const int32_t *>(smem + C::OFF_PAGES);
    const int pblk = PAGED ? a.pt.page_rows / kBlockRows : 1;
    if constexpr (PAGED) {
        // every block of every tile (the last tile may reach one block past
        // nrows), within the table
        const int64_t trows = (int64_t)ntiles * kTileRows < nblocks_plane * kBlockRows
                                  ? (int64_t)ntiles * kTileRows : nblocks_plane * kBlockRows;
        const int npages = (int)((trows + a.pt.page_rows - 1) / a.pt.page_rows);
        int32_t *dst = reinterpret_cast<int32_t *>(smem + C::OFF_PAGES);
        for (int i = tid; i < npages; i += C::THREADS) dst[i] = a.pt.table[(int64_t)a.seq * a.pt.table_stride + i];
    }
    // Where block gb of the sequence lives: code and scale pointers of each
    // plane; false when its page entry points outside the pool (the block
    // then reads as zeros).
    auto block_at = [&](int64_t gb, const uint8_t *&kc, const uint8_t *&vc, const uint16_t *&ks,
                        const uint16_t *&vs) -> bool {
        if constexpr (!PAGED) {
            kc = kcodes + gb * C::K_BLOCK_BYTES;
            vc = vcodes + gb * C::V_BLOCK_BYTES;
            ks = kscales + gb * C::K_BLOCK_SCALES;
            vs = vscales + gb * C::V_BLOCK_SCALES;
            return true;
        } else {
            const PageSlot ps = page_slot(gb, pblk);
            const int page = page_lds[ps.entry];
            if (page < 0 || page >= a.k.n_seqs) return false;
            const int64_t hl = (int64_t)page * a.k.n_kv_heads + kvh;
            const int64_t within = ps.within;
            kc = a.k.codes + hl * a.k.head_code_stride + within * C::K_BLOCK_BYTES;
            vc = a.v.codes + hl * a.v.head_code_stride + within * C::V_BLOCK_BYTES;
            ks = a.k.scales + hl * a.k.head_scale_stride + within * C::K_BLOCK_SCALES;
            vs = a.v.scales + hl * a.v.head_scale_stride + within * C::V_BLOCK_SCALES;
            return true;
        }
    };

    // The tile pipeline: a tile's codes are loaded into registers and its
    // scales staged in LDS one iteration before it is dequantized, which is
    // one iteration before its products, so neither the global loads nor the
    // dequant wait in line with the matrix products.
    uint32_t rk[C::UK][C::K_UW / 4], rv[C::UV][C::V_UW / 4];
    u4 rsc = u4{0u, 0u, 0u, 0u};
    uint16_t *sc_lds = reinterpret_cast<uint16_t *>(lds + C::OFF_SC);  // [2][SC_BYTES / 2]
    // a tile's code words into this thread's registers
    auto load_codes = [&](int tile) {
        const int64_t b0 = (int64_t)tile * 2;  // first block of the tile
        const bool two = b0 + 1 < nblocks_plane;  // the second block exists
        if constexpr (!PAGED) {
            // contiguous planes: the tile's two blocks are adjacent
            const uint8_t *kb = kcodes + b0 * C::K_BLOCK_BYTES;
            const uint8_t *vb = vcodes + b0 * C::V_BLOCK_BYTES;
#pragma unroll
            for (int i = 0; i < C::UK; ++i) {
                const int u = tid + i * C::THREADS;
                if (u < C::K_UNITS && (two || u < C::K_UNITS / 2))
                    load_chunk<C::K_UW>(rk[i], kb + k_unit_offset<D, KC, VC>(u));
            }
#pragma unroll
            for (int i = 0; i < C::UV; ++i) {
                const int u = tid + i * C::THREADS;
                if (u < C::V_UNITS && (two || u < C::V_UNITS / 2))
                    load_chunk<C::V_UW>(rv[i], vb + v_unit_offset<D, KC, VC>(u));
            }
            return;
        }
        // paged: each block's planes (a tile's two blocks may sit in
        // different pages); an absent second block is never read.  The two
        // blocks' pointers are picked by a select, not from an array indexed
        // per lane: through such an array the compiler loses track of the
        // address space and issues flat loads, which count against the LDS
        // wait counter too, so every LDS operand wait behind them would also
        // wait for these loads to land.
        const uint8_t *kb0, *vb0, *kb1 = nullptr, *vb1 = nullptr;
        const uint16_t *ksb, *vsb;
        const bool ok0 = block_at(b0, kb0, vb0, ksb, vsb);
        const bool ok1 = two && block_at(b0 + 1, kb1, vb1, ksb, vsb);
#pragma unroll
        for (int i = 0; i < C::UK; ++i) {
            const int u = tid + i * C::THREADS;
            if (u >= C::K_UNITS) continue;
            const bool j = u >= C::K_UNITS / 2;  // units of block 0 come first
            if (j ? ok1 : ok0)
                load_chunk<C::K_UW>(rk[i], (j ? kb1 : kb0) + (k_unit_offset<D, KC, VC>(u) - (j ? C::K_BLOCK_BYTES : 0)));
            else
#pragma unroll
                for (int w = 0; w < C::K_UW / 4; ++w) rk[i][w] = 0u;
        }
#pragma unroll
        for (int i = 0; i < C::UV; ++i) {
            const int u = tid + i * C::THREADS;
            if (u >= C::V_UNITS) continue;
            const bool j = u >= C::V_UNITS / 2;
            if (j ? ok1 : ok0)
                load_chunk<C::V_UW>(rv[i], (j ? vb1 : vb0) + (v_unit_offset<D, KC, VC>(u) - (j ? C::V_BLOCK_BYTES : 0)));
            else
#pragma unroll
                for (int w = 0; w < C::V_UW / 4; ++w) rv[i][w] = 0u;
        }
    };
    // a tile's scales, 16 bytes per thread of the first SC_BYTES / 16: K (both
    // blocks) then V; under paging a block outside the pool gets zero scales
    auto load_scales = [&](int tile) {
        const int o = tid * 16;
        if (o >= C::SC_BYTES) return;
        const int64_t b0 = (int64_t)tile * 2;
        const bool two = b0 + 1 < nblocks_plane;
        if constexpr (!PAGED) {
            if (o < C::KSC_BYTES) {
                if (two || o < C::KSC_BYTES / 2)
                    rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(kscales + b0 * C::K_BLOCK_SCALES) + o);
            } else {
                const int ov = o - C::KSC_BYTES;
                if (two || ov < C::VSC_BYTES / 2)
                    rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(vscales + b0 * C::V_BLOCK_SCALES) + ov);
            }
            return;
        }
        const uint8_t *kb, *vb;
        const uint16_t *ksb, *vsb;
        if (o < C::KSC_BYTES) {
            const int j = o >= C::KSC_BYTES / 2, oj = o - j * (C::KSC_BYTES / 2);
            const bool ok = (j == 0 || two) && block_at(b0 + j, kb, vb, ksb, vsb);
            if (ok) rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(ksb) + oj);
            else rsc = u4{0u, 0u, 0u, 0u};
        } else {
            const int ov = o - C::KSC_BYTES;
            const int j = ov >= C::VSC_BYTES / 2, oj = ov - j * (C::VSC_BYTES / 2);
            const bool ok = (j == 0 || two) && block_at(b0 + j, kb, vb, ksb, vsb);
            if (ok) rsc = *reinterpret_cast<const u4 *>(reinterpret_cast<const uint8_t *>(vsb) + oj);
            else rsc = u4{0u, 0u, 0u, 0u};
        }
    };
    auto load_tile = [&](int tile) {
        load_codes(tile);
        load_scales(tile);
    };
    auto stage_scales = [&](int tile) {
        if (tid * 16 < C::SC_BYTES)
            *reinterpret_cast<u4 *>(reinterpret_cast<uint8_t *>(sc_lds + (tile & 1) * (C::SC_BYTES / 2)) + tid * 16) = rsc;
    };
    // dequantizes the tile whose codes are in rk/rv and whose scales are staged
    auto dequant_tile = [&](int tile, f16bits *khat, f16bits *vhat) {
        const int64_t b0 = (int64_t)tile * 2;
        const int vrows = (int)min((int64_t)kTileRows, nrows - (int64_t)tile * kTileRows);
        const bool two = b0 + 1 < nblocks_plane;
        const uint16_t *ksc = sc_lds + (tile & 1) * (C::SC_BYTES / 2);
        const uint16_t *vsc = ksc + C::KSC_BYTES / 2;
#pragma unroll
        for (int i = 0; i < C::UK; ++i) {
            const int u = tid + i * C::THREADS;
            if (u >= C::K_UNITS || (!two && u >= C::K_UNITS / 2)) continue;  // block 1 absent: rows unused
            deq_k_unit<D, KC, VC>(u, rk[i], ksc, khat);
        }
#pragma unroll
        for (int i = 0; i < C::UV; ++i) {
            const int u = tid + i * C::THREADS;
            if (u >= C::V_UNITS) continue;
            if (!two && u >= C::V_UNITS / 2) {
                // absent block: zero its V columns so masked products stay 0
                const VUnit vu = v_unit<D, KC, VC>(u);
                const int c16 = vu.L & 15, kq = vu.L >> 4;
                constexpr int CBS = C::V_UW / C::V_BPC;
                const int cb0 = (vu.c * C::V_CW + vu.sub * C::V_UW) / C::V_BPC;
#pragma unroll
                for (int k = 0; k < CBS; ++k) {
                    f16bits *dst = vhat + (16 * (cb0 + k) + c16) * C::VS + 32 + 4 * kq;
                    *reinterpret_cast<u2 *>(dst) = u2{0u, 0u};
                    *reinterpret_cast<u2 *>(dst + 16) = u2{0u, 0u};
                }
                continue;
            }
            deq_v_unit<D, KC, VC>(u, rv[i], vsc, vhat, vrows < kTileRows, vrows);
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

    auto kbuf = [&](int tile) { return lds + (tile & 1) * C::K_TILE_ELEMS; };
    auto vbuf = [&](int tile) { return lds + C::OFF_V + (tile % C::NVB) * C::V_TILE_ELEMS; };

    // ---- S^T = K_hat Q^T for one tile: 4 row tiles x NT column tiles
    f4 S[C::NT][4];
    auto scores = [&](int tile) {
        const f16bits *khat = kbuf(tile);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            h8 kop[C::KSTEPS];
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks)
                kop[ks] = *reinterpret_cast<const h8 *>(khat + (16 * mt + h16) * C::KS + 32 * ks + 8 * q4);
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) {
                f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < C::KSTEPS; ++ks) acc = mfma16x16x32(kop[ks], qop[nt][ks], acc);
                S[nt][mt] = acc;  // unscaled: the column's factor enters with the exponent
            }
        }
    };
    // ---- masking and the online-softmax update of one tile's scores; the
    // probabilities become the P^T operands (k-step ks covers row tiles
    // 2ks, 2ks+1)
    h8 P[C::NT][2];
    auto softmax = [&](int tile) {
        const int row0 = tile * kTileRows;
        const bool diag_tile = row0 + kTileRows - 1 > wave_min_diag;
        // the column maxima of all column tiles first, so that their
        // cross-lane stages overlap, then one rescale decision for the wave
        float mx[C::NT];
        bool raise[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
            if (diag_tile) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (row0 + 16 * mt + 4 * q4 + r > diag[nt]) S[nt][mt][r] = -INFINITY;
            }
            mx[nt] = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx[nt] = fmaxf(mx[nt], S[nt][mt][r]);
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) mx[nt] = swap_max16(mx[nt]);
        bool any_raise = false;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
            // (the two lane-swap stages of all column tiles are interleaved)
            mx[nt] = swap_max32(mx[nt]) * cscale[nt];  // -inf stays -inf (the factor is positive)
            // a column with every row of this tile masked keeps its state
            raise[nt] = mx[nt] > m_run[nt] + kPRescaleThreshold;
            any_raise |= raise[nt];
        }
        if (__any(any_raise)) {
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt) {
                const float m_new = raise[nt] ? mx[nt] : m_run[nt];
                const float alpha = raise[nt] ? fast_exp2(m_run[nt] - m_new) : 1.0f;
                l_run[nt] *= alpha;
#pragma unroll
                for (int cb = 0; cb < C::CB; ++cb) O[nt][cb] *= alpha;
                m_run[nt] = m_new;
            }
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)  // 0 when masked
                    P[nt][mt >> 1][4 * (mt & 1) + r] = (_Float16)fast_exp2(fmaf(S[nt][mt][r], cscale[nt], -m_run[nt]));
            // the row sum takes the binary16 probabilities the PV product
            // uses, two per dot-product instruction (exact products by 1,
            // fp32 sum)
            const h2 one = h2{(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    l_run[nt] = __builtin_amdgcn_fdot2(h2{P[nt][ks][2 * j], P[nt][ks][2 * j + 1]}, one, l_run[nt], false);
        }
    };
    // ---- O^T += V_hat^T P^T; each V_hat operand read serves every column
    // tile of the wave
    auto pv = [&](int tile) {
        const f16bits *vhat = vbuf(tile);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16bits *vp = vhat + (16 * cb + h16) * C::VS + 32 * ks + 4 * q4;
                const u2 lo = *reinterpret_cast<const u2 *>(vp);
                const u2 hi = *reinterpret_cast<const u2 *>(vp + 16);
                const h8 vop = __builtin_bit_cast(h8, u4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt) O[nt][cb] = mfma16x16x32(vop, P[nt][ks], O[nt][cb]);
            }
        }
    };

    // prologue: tile 0 dequantized, tile 1 loaded and its scales staged
    if constexpr (PAGED) __syncthreads();  // the page numbers are in LDS
    load_tile(0);
    stage_scales(0);
    __syncthreads();
    dequant_tile(0, kbuf(0), vbuf(0));
    if (1 < ntiles) {
        load_tile(1);
        stage_scales(1);
    }
    __syncthreads();
    // Each tile passes through S (matrix cores), softmax (vector ALU) and PV
    // (matrix cores).  Waves 0-3 run PV(k-1), S(k), softmax(k) between the
    // barriers of iteration k; waves 4-7 (the other wave of each SIMD) run
    // softmax(k-1), PV(k-1), S(k): the two waves of a SIMD then use the matrix
    // cores and the vector ALU at the same time instead of in lockstep.  A
    // tile's V_hat is therefore read one iteration after its K_hat (three
    // V_hat buffers).  Without room for three, every wave runs S(k),
    // softmax(k), PV(k).
    const bool late = C::PINGPONG && wave >= C::WAVES / 2;
    bool have_s = false;  // S holds the scores of tile - 1 (late waves)
    bool have_p = false;  // P holds the probabilities of tile - 1
    for (int tile = 0; tile < ntiles; ++tile) {
        // the late waves dequantize the next tile first (their matrix phase
        // comes last), the early ones last (theirs comes first), so a SIMD's
        // two waves overlap vector and matrix work in both halves
        if (late || !C::PINGPONG) {
            if (tile + 1 < ntiles) dequant_tile(tile + 1, kbuf(tile + 1), vbuf(tile + 1));
            if (tile + 2 < ntiles) {
                if constexpr (!C::PINGPONG) loads_landed();
                load_tile(tile + 2);
            }
        } else if (tile + 2 < ntiles) {
            // the early waves hold the staging threads: their scale loads
            // go out first, so that the staging at the end of the iteration
            // does not wait a memory round trip in front of the barrier
            load_scales(tile + 2);
        }
        if (late && have_s) {
            softmax(tile - 1);
            have_s = false;
            have_p = true;
        }
        // some column of this wave sees rows of this tile (false from some
        // tile on, for every later one)
        const bool act = tile * kTileRows <= wave_max_diag;
        if (act && have_p) {
            // the usual case: the products of the previous tile's PV and of
            // this tile's scores are independent, and in one block the
            // scheduler can hide each stream's LDS operand reads behind the
            // other's matrix products (PV first measured faster)
            pv(tile - 1);
            scores(tile);
            reads_ahead_of_products<C::CB * 2 + 4 * C::KSTEPS, C::CB * 2 * C::NT + 4 * C::NT * C::KSTEPS, read_lead<D>()>();
            have_p = false;
        } else {
            if (act) {
                scores(tile);
                reads_ahead_of_products<4 * C::KSTEPS, 4 * C::NT * C::KSTEPS, read_lead<D>()>();
            }
            if (have_p) {
                pv(tile - 1);
                reads_ahead_of_products<C::CB * 2, C::CB * 2 * C::NT, read_lead<D>()>();
                have_p = false;
            }
        }
        if (act) {
            if (late) {
                have_s = true;
            } else {
                softmax(tile);
                if constexpr (C::PINGPONG) have_p = true;
                else {
                    pv(tile);
                    reads_ahead_of_products<C::CB * 2, C::CB * 2 * C::NT, read_lead<D>()>();
                }
            }
        }
        if (!late && C::PINGPONG) {
            if (tile + 1 < ntiles) dequant_tile(tile + 1, kbuf(tile + 1), vbuf(tile + 1));
            if (tile + 2 < ntiles) load_codes(tile + 2);
        }
        // tile + 2's scales go where tile's were (read by its dequant, one
        // iteration ago); the staging threads (wave 0) loaded them at the top
        // of this iteration
        if (tile + 2 < ntiles) stage_scales(tile + 2);
        __syncthreads();  // next tile's dequant and staging done; this tile's reads done
    }
    if (have_s) {
        softmax(ntiles - 1);
        have_p = true;
    }
    if (have_p) pv(ntiles - 1);

    // ---- normalize and store: lane (column h16, q4) holds channels 16cb+4q4..+3.
    // A K_hat or V_hat beyond the binary16 range (|code * dq| > 65504) became
    // an infinity in LDS, which reaches every output it can affect as an
    // infinity or a NaN (0 * inf included); only a causally masked row drops
    // out, and then the result is right.  So a non-finite output marks the
    // call as outside the operand range (finite queries assumed).
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
        const float L = quad_sum(l_run[nt]);
        if (diag[nt] < 0) continue;
        const int col = col0 + (wave * C::NT + nt) * 16 + h16;
        const int t = col / G, hh = col % G;
        float *dst = a.out + ((int64_t)t * a.n_q_heads + (int64_t)kvh * G + hh) * D;
        const float inv = 1.0f / L;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const f4 o = O[nt][cb] * inv;
            bad |= !(__builtin_isfinite(o[0]) && __builtin_isfinite(o[1]) && __builtin_isfinite(o[2]) &&
                     __builtin_isfinite(o[3]));
            *reinterpret_cast<f4 *>(dst + 16 * cb + 4 * q4) = o;
        }
    }
    if (a.dev_status && __any(bad) && lane == 0) *a.dev_status = kStatusOverflow;
}

template <int D, int KC, int VC, bool PAGED>
hipError_t launch_ptyped_p(const PrefillArgs &a, hipStream_t s) {
    using C = PCfg<D, KC, VC, PAGED>;
    const size_t lds = (size_t)C::LDS_BYTES;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_kernel<D, KC, VC, PAGED>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int ncols = a.n_tokens * a.gqa;
    const dim3 grid((unsigned)((ncols + C::COLS - 1) / C::COLS * a.k.n_kv_heads));
    prefill_kernel<D, KC, VC, PAGED><<<grid, dim3(C::THREADS), lds, s>>>(a);
    return hipGetLastError();
}

template <int D, int KC, int VC>
hipError_t launch_ptyped(const PrefillArgs &a, hipStream_t s) {
    return a.pt.table ? launch_ptyped_p<D, KC, VC, true>(a, s) : launch_ptyped_p<D, KC, VC, false>(a, s);
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
    // the block codecs (the f16 control codec is a decode-only baseline)
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
