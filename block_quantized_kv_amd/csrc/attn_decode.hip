// attn_decode.hip -- split-K decode attention over the block-quantized cache,
// plus the log-sum-exp combine of the splits.  gfx950.
//
// What is computed (den_llama.cpp, "Results" / "What's in the fork":
// FlashAttention reads the q8_0 / q4_0 / Q4_G64 K and V blocks directly;
// "Ship command": up to two drafted tokens are verified per step): for each
// of the q_len newest positions p_i = len_b - q_len + i,
//   out[b][i][h] = sum_{j <= p_i} softmax_j(scale * q[b][i][h] . k_hat_j) v_hat_j
// over kv-head h / gqa (q_len = 1 is plain decode).
//
// Design (one workgroup = 8 waves = one split of `split_rows` rows of one
// (sequence, kv-head); the waves share the split's 32-row blocks):
//  * The GQA group times the queries per sequence (<= 16 columns, each a
//    (query, head) pair) is the N side of 16x16x32 f16 matrix products, so
//    every K/V byte is read once per kv-head for all of them:
//      S^T[row][head] = K[row][:] . Q'[:][head]   (A = K codes, B = query)
//      O^T[ch][head] += V[ch][rows] . P^T[rows][head]
//    The accumulator layout of S^T (lane = head + 16*q holds rows 4q..4q+3 of
//    each 16-row tile) is exactly the B-operand layout P^T needs, and the
//    V-role block layout puts each lane's eight V rows where its probabilities
//    are, so no data moves between the two products.
//  * K codes enter the matrix cores as exact binary16 "1024 + n" / "1152 + b"
//    values (one bit-select per pair, or a byte permute); the constant bias is
//    cancelled by starting the accumulator at -sum(query * bias).  The query
//    is scaled by a power of two and split into hi + lo binary16 halves (two
//    products), so the score keeps ~22 bits.  K group scales are applied in
//    fp32 to each group's partial dot product.  Both 16-row tiles of a block
//    walk the channel steps together (two independent accumulator chains).
//  * V enters as binary16 code * dq (one rounding, exact for subnormal dq);
//    probabilities enter as binary16.  Statistics and sums are fp32.
//  * Online softmax in log2 units; the running max is only raised when a
//    block exceeds it by more than 8 (probabilities stay <= 256), so the
//    rescale of O is rare.
//  * Streaming: blocks travel HBM -> LDS by buffer-to-LDS DMA, which holds no
//    registers while in flight.  Each wave owns a ring of NS block slots in
//    LDS (byte layout = the cache's); it copies the oldest slot into
//    registers, immediately refills that slot with the next block of the
//    split (handed out by an LDS counter, so fast waves take more) and
//    computes from the registers, so NS blocks per wave are always on their
//    way.  NS keeps about 72 KB per workgroup in flight: deeper rings only
//    lengthen the memory queues.  The compiler cannot see which LDS bytes a DMA writes (it
//    would wait for every DMA before any LDS read), so the slot reads are
//    hand-issued with an explicit wait for exactly the DMAs of that slot.
//    Every DMA is issued unconditionally: one past the end of the split is
//    cut off by the buffer range check and touches no memory.  The DMAs are
//    non-temporal (each K/V byte is read once per call).  A one-block ring
//    starts with two blocks per wave where LDS has room (head start); big
//    head_dim 256 blocks are copied and consumed K half, then V half.
//  * The query operand (hi/lo halves for every channel step) and the bias
//    corrections are prepared once per workgroup, each wave taking one channel
//    step, and shared through LDS.
//  * Fused append: the workgroup whose split holds the step's new rows
//    quantizes and stores them first (wave 0); DMAs of the blocks those
//    stores touch wait for them (an LDS flag where possible, else a barrier).
//  * The 8 waves merge through LDS: each parks its unscaled O and (max, sum)
//    in its own slots as soon as its blocks are done, and after one barrier
//    each thread weighs the 8 copies (or, where the parked columns do not
//    fit, rescale to the common max, then sum).  Each workgroup writes one
//    partial (unnormalized O, max, sum) per query head, or the final output
//    when the sequence fits in one split; combine_kernel merges the splits
//    (log-sum-exp) with many partial loads in flight at once.
#include <mutex>
#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_quant.h"

namespace kvq {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 160 * 1024;  // per workgroup on gfx950
constexpr float kRescaleThreshold = 8.0f;
constexpr int kInflightBytes = 72 * 1024;  // target DMA bytes in flight per workgroup

// number of DMA instructions that copy a region of B bytes (1 KB per dwordx4
// DMA, 256 B per dword DMA, a lane-masked dword DMA for a shorter tail)
constexpr int dma_count(int B) { return B / 1024 + (B % 1024) / 256 + ((B % 256) ? 1 : 0); }

template <int D, int KC, int VC>
struct Cfg {
    static constexpr int KSTEPS = D / 32;
    // f16 K has no scales: one "group" spans the row (scale 1)
    static constexpr int KG = is16(KC) ? D : group_size(KC);
    static constexpr int KNG = D / KG;
    static constexpr int STEPS_PER_KGROUP = KG / 32;
    static constexpr int VG = group_size(VC);
    static constexpr int VNG = is16(VC) ? 0 : D / VG;
    // words per k-step (K) and per 16-channel block (V) of one lane
    static constexpr int K_WPS = is16(KC) ? 4 : is8(KC) ? 2 : 1;
    static constexpr int V_WPC = is16(VC) ? 4 : is8(VC) ? 2 : 1;
    static constexpr int CB = D / 16;
    static constexpr int K_LB = k_lane_bytes(KC, D);      // bytes per lane per K tile
    static constexpr int V_LB = v_lane_bytes(VC, D);      // bytes per lane per V block
    static constexpr int K_W = chunk_width(K_LB);
    static constexpr int V_W = chunk_width(V_LB);
    static constexpr int K_WORDS = K_LB / 4;
    static constexpr int V_WORDS = V_LB / 4;
    static constexpr int K_TILE_BYTES = 16 * row_bytes(KC, D);
    static constexpr int K_BLOCK_BYTES = block_code_bytes(KC, D);
    static constexpr int V_BLOCK_BYTES = block_code_bytes(VC, D);
    static constexpr int K_BLOCK_SCALES = block_scales(KC, D);
    static constexpr int V_BLOCK_SCALES = block_scales(VC, D);
    // one block slot in LDS: [K codes][V codes][K scales][V scales]
    static constexpr int SL_K = 0;
    static constexpr int SL_V = SL_K + K_BLOCK_BYTES;
    static constexpr int SL_KS = SL_V + V_BLOCK_BYTES;
    static constexpr int SL_VS = SL_KS + 2 * K_BLOCK_SCALES;
    static constexpr int SLOT = SL_VS + 2 * V_BLOCK_SCALES;
    static constexpr int N_DMA_K = dma_count(K_BLOCK_BYTES) + dma_count(2 * K_BLOCK_SCALES);
    static constexpr int N_DMA_V = dma_count(V_BLOCK_BYTES) + dma_count(2 * V_BLOCK_SCALES);
    static constexpr int N_DMA = N_DMA_K + N_DMA_V;
    // per-lane scale words of one block: K (4 rows x KNG groups per tile),
    // V (8 rows x VNG groups)
    static constexpr int KS_LANE_BYTES = is16(KC) ? 0 : 8 * KNG;   // per tile
    static constexpr int VS_LANE_BYTES = 16 * VNG;
    // head_dim 256: the query operand is read from LDS at every channel step,
    // leaving the registers to the output accumulator and one block
    static constexpr bool Q_LDS = D == 256;
    // LDS layout (bytes); the final merge reuses it
    static constexpr int OFF_QOP = 0;                                 // [KSTEPS][hi,lo][64 lanes] h8
    static constexpr int OFF_TMAX = OFF_QOP + KSTEPS * 2 * 64 * 16;   // [KSTEPS][16] fp32
    static constexpr int OFF_CORR = OFF_TMAX + KSTEPS * 16 * 4;       // [KSTEPS][16] fp32
    static constexpr int OFF_CNT = OFF_CORR + KSTEPS * 16 * 4;        // block hand-out counter, append flag
    static constexpr int OFF_ML = OFF_CNT + 16;                       // [wave][16] (max, sum)
    static constexpr int OFF_FIN = OFF_ML + kWaves * 16 * 8;          // [16] merged (max, sum)
    static constexpr int OFF_SLOTS = OFF_FIN + 16 * 8;                // [wave][NS] slots
    // Ring depth: about 72 KB of blocks in flight per compute unit.  More
    // only lengthens the memory queues (and the spread of completion times
    // at the end of a split) without raising the streaming rate: at 64K
    // context a one-block ring (70 KB) beats two (140 KB) by ~10%.
    static constexpr int NS_FIT = (kLdsBytes - OFF_SLOTS) / (kWaves * SLOT);
    static constexpr int NS_TGT = kInflightBytes / (kWaves * SLOT) < 1 ? 1 : kInflightBytes / (kWaves * SLOT);
    static constexpr int NS = NS_TGT < NS_FIT ? (NS_TGT < 3 ? NS_TGT : 3) : NS_FIT;
    // Blocks whose one-lane share is 80 words or more at head_dim 256 (8-bit
    // codes, or q4_0 K with its 8 scale groups) are read in two halves: the K
    // half is copied, refilled and scored before the V half is copied, so
    // both are never held in registers at once (the single copy spills)
    static constexpr int NWK = 2 * K_WORDS + KS_LANE_BYTES / 2;
    static constexpr int NWV = V_WORDS + VS_LANE_BYTES / 4;
    static constexpr bool TWO_PHASE = NS == 1 && NWK + NWV >= 80 && D == 256;
    // A one-block ring starts with two blocks per wave when LDS allows: the
    // wave then has its second block on the way while it computes its first,
    // instead of requesting it only once the first has arrived.
    static constexpr bool HEAD2 = NS == 1 && NS_FIT >= 2 && !TWO_PHASE;
    static constexpr int NSLOT = NS + (HEAD2 ? 1 : 0);  // slots per wave
    // A block's code bytes are always whole 128-byte lines; its scales are
    // too except for Q4_G64 at head_dim 64 (64 bytes), where a line of scales
    // is shared with a neighbouring block
    static constexpr bool SCALES_WHOLE_LINES = (2 * K_BLOCK_SCALES) % 128 == 0 && (2 * V_BLOCK_SCALES) % 128 == 0;
    static_assert(NS >= 1, "one block slot per wave must fit in LDS");
    static_assert((NS - 1) * N_DMA <= 63, "DMAs in flight exceed the wait counter");
    static_assert(SL_V % 16 == 0 && SL_KS % 16 == 0 && SL_VS % 16 == 0 && SLOT % 16 == 0, "slot alignment");
    static_assert(NSLOT * SLOT <= 65535, "slot offsets fit the DS immediate");
    static constexpr int LDS_STREAM = OFF_SLOTS + kWaves * NSLOT * SLOT;
    // the final merge parks every wave's output columns, DP floats apart
    // (D + 16: conflict-free 16-byte writes), from OFF_SLOTS on
    static constexpr int DP = D + 16;
    static constexpr int LDS_MERGE_MAX = OFF_SLOTS + kWaves * 16 * DP * 4;
    static_assert(LDS_MERGE_MAX <= kLdsBytes, "the merge fits in LDS");
};

// Raw buffer descriptor (base in SGPRs, byte range checked by the hardware).
// The whole byte offset goes in the VGPR offset, which the range check covers:
// a DMA of a block past the end of the split touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

struct Streams {
    __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
};

typedef __attribute__((address_space(3))) void lds_void;

// Cache policy of the block DMAs: non-temporal.  Every K/V byte is read once
// per call, so the lines are not worth keeping; measured 22.4 -> 20.9 us per
// 64K step and 238 -> 222 us per 196K four-layer step.
constexpr int kStreamPolicy = 2;  // nt

// Copies B bytes at byte goff of stream r to LDS at dst (a plain copy; lane
// l carries bytes [16 l, 16 l + 16) of each 1 KB piece).
template <int B>
__device__ __forceinline__ void dma_region(__amdgpu_buffer_rsrc_t r, uint32_t goff, unsigned char *dst, int lane) {
    constexpr int N16 = B / 1024, N4 = (B % 1024) / 256, TAIL = B % 256;
#pragma unroll
    for (int c = 0; c < N16; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + c * 1024), 16, goff + c * 1024 + lane * 16, 0, 0, kStreamPolicy);
#pragma unroll
    for (int c = 0; c < N4; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + N16 * 1024 + c * 256), 4,
                                                 goff + N16 * 1024 + c * 256 + lane * 4, 0, 0, kStreamPolicy);
    if constexpr (TAIL != 0) {
        static_assert(TAIL % 4 == 0, "scale regions are whole words");
        if (lane * 4 < TAIL)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + N16 * 1024 + N4 * 256), 4,
                                                     goff + N16 * 1024 + N4 * 256 + lane * 4, 0, 0, kStreamPolicy);
    }
}

// The K half (codes, scales) or the V half of block idx, as one DMA group.
template <int D, int KC, int VC>
__device__ __forceinline__ void dma_half(const Streams &st, int idx, unsigned char *slot, int lane, bool k_half) {
    using C = Cfg<D, KC, VC>;
    if (k_half) {
        dma_region<C::K_BLOCK_BYTES>(st.kc, (uint32_t)idx * C::K_BLOCK_BYTES, slot + C::SL_K, lane);
        dma_region<2 * C::K_BLOCK_SCALES>(st.ks, (uint32_t)idx * C::K_BLOCK_SCALES * 2, slot + C::SL_KS, lane);
    } else {
        dma_region<C::V_BLOCK_BYTES>(st.vc, (uint32_t)idx * C::V_BLOCK_BYTES, slot + C::SL_V, lane);
        dma_region<2 * C::V_BLOCK_SCALES>(st.vs, (uint32_t)idx * C::V_BLOCK_SCALES * 2, slot + C::SL_VS, lane);
    }
}

// Both halves, K first.
template <int D, int KC, int VC>
__device__ __forceinline__ void dma_block(const Streams &st, int idx, unsigned char *slot, int lane) {
    using C = Cfg<D, KC, VC>;
    dma_half<D, KC, VC>(st, idx, slot, lane, true);
    dma_half<D, KC, VC>(st, idx, slot, lane, false);
}

// ---- hand-issued LDS reads (no wait; see lds_wait).  `off` must fold to a
// constant after inlining and unrolling (it becomes the DS immediate).
__device__ __forceinline__ void ds_rd(u4 &x, uint32_t a, int off) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(off) : "memory");
}
__device__ __forceinline__ void ds_rd(u2 &x, uint32_t a, int off) {
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(off) : "memory");
}
__device__ __forceinline__ void ds_rd(uint32_t &x, uint32_t a, int off) {
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(x) : "v"(a), "i"(off) : "memory");
}
// Reads the LB bytes a lane owns at byte offset `off` of an LDS copy of a
// chunk-major region into words (a16/a8/a4: region base + lane * width).
template <int LB>
__device__ __forceinline__ void ds_rd_lane(uint32_t *w, uint32_t a16, uint32_t a8, uint32_t a4, int off) {
    constexpr int W = chunk_width(LB);
    if constexpr (W == 16) {
#pragma unroll
        for (int c = 0; c < LB / 16; ++c) {
            u4 v;
            ds_rd(v, a16, off + c * 1024);
            w[4 * c + 0] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
        }
    } else if constexpr (W == 8) {
        u2 v;
        ds_rd(v, a8, off);
        w[0] = v.x; w[1] = v.y;
    } else {
        ds_rd(w[0], a4, off);
    }
}
// Reads NB contiguous bytes (a multiple of 8) at a + off into words.
template <int NB>
__device__ __forceinline__ void ds_rd_span(uint32_t *w, uint32_t a, int off) {
#pragma unroll
    for (int c = 0; c < NB / 16; ++c) {
        u4 v;
        ds_rd(v, a, off + c * 16);
        w[4 * c + 0] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
    }
    if constexpr (NB % 16 == 8) {
        u2 v;
        ds_rd(v, a, off + (NB / 16) * 16);
        w[4 * (NB / 16)] = v.x;
        w[4 * (NB / 16) + 1] = v.y;
    }
}
__device__ __forceinline__ void ds_wr(uint32_t a, uint32_t x, int off) {
    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(a), "v"(x), "i"(off) : "memory");
}
__device__ __forceinline__ void ds_wr(uint32_t a, u4 x, int off) {
    asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(a), "v"(x), "i"(off) : "memory");
}
// Atomic add on an LDS word, returning the old value (waits for it).
__device__ __forceinline__ uint32_t ds_add_rtn(uint32_t a, uint32_t x, int off) {
    uint32_t r;
    asm volatile("ds_add_rtn_u32 %0, %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a), "v"(x), "i"(off) : "memory");
    return r;
}
// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its memory loads (a __syncthreads would also wait for every DMA).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Completes the hand-issued LDS reads: waits for them and makes every word
// read so far a fresh value for the compiler (N words).
template <int N>
__device__ __forceinline__ void lds_wait(uint32_t *w) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(w[i]));
}
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Buffer descriptors of one block of a paged plane pair: block `within` of
// page `page` (records 0, so every access is cut off, for page < 0).
template <int D, int KC, int VC>
__device__ __forceinline__ Streams page_block_streams(const DecodeArgs &a, int page, int kvh, int within) {
    using C = Cfg<D, KC, VC>;
    const bool ok = page >= 0 && page < a.k.n_seqs;
    const int64_t hl = ok ? (int64_t)page * a.k.n_kv_heads + kvh : 0;
    Streams st;
    st.kc = make_rsrc(a.k.codes + hl * a.k.head_code_stride + (int64_t)within * C::K_BLOCK_BYTES,
                      ok ? C::K_BLOCK_BYTES : 0);
    st.vc = make_rsrc(a.v.codes + hl * a.v.head_code_stride + (int64_t)within * C::V_BLOCK_BYTES,
                      ok ? C::V_BLOCK_BYTES : 0);
    st.ks = make_rsrc(a.k.scales + hl * a.k.head_scale_stride + (int64_t)within * C::K_BLOCK_SCALES,
                      ok ? C::K_BLOCK_SCALES * 2 : 0);
    st.vs = make_rsrc(a.v.scales + hl * a.v.head_scale_stride + (int64_t)within * C::V_BLOCK_SCALES,
                      ok ? C::V_BLOCK_SCALES * 2 : 0);
    return st;
}

// One block's words for one lane, copied out of its LDS slot.
template <int D, int KC, int VC>
struct Payload {
    using C = Cfg<D, KC, VC>;
    static constexpr int NW = C::NWK + C::NWV;  // [K tiles][K scales] [V][V scales]
    uint32_t w[NW];
    __device__ __forceinline__ uint32_t *k(int tau) { return w + tau * C::K_WORDS; }
    __device__ __forceinline__ uint32_t *ks(int tau) { return w + 2 * C::K_WORDS + tau * (C::KS_LANE_BYTES / 4); }
    __device__ __forceinline__ uint32_t *v() { return w + C::NWK; }
    __device__ __forceinline__ uint32_t *vs() { return w + C::NWK + C::V_WORDS; }
};

template <int D, int KC, int VC>
__device__ __forceinline__ void read_slot(Payload<D, KC, VC> &pl, uint32_t a16, uint32_t a8, uint32_t a4,
                                          uint32_t aks, uint32_t avs, int soff) {
    using C = Cfg<D, KC, VC>;
    ds_rd_lane<C::K_LB>(pl.k(0), a16, a8, a4, soff + C::SL_K);
    ds_rd_lane<C::K_LB>(pl.k(1), a16, a8, a4, soff + C::SL_K + C::K_TILE_BYTES);
    ds_rd_lane<C::V_LB>(pl.v(), a16, a8, a4, soff + C::SL_V);
    ds_rd_span<C::KS_LANE_BYTES>(pl.ks(0), aks, soff + C::SL_KS);
    ds_rd_span<C::KS_LANE_BYTES>(pl.ks(1), aks, soff + C::SL_KS + 32 * C::KNG);
    ds_rd_span<C::VS_LANE_BYTES>(pl.vs(), avs, soff + C::SL_VS);
    lds_wait<Payload<D, KC, VC>::NW>(pl.w);
}
// The K half alone (codes of both tiles and their scales) ...
template <int D, int KC, int VC>
__device__ __forceinline__ void read_slot_k(Payload<D, KC, VC> &pl, uint32_t a16, uint32_t a8, uint32_t a4,
                                            uint32_t aks, int soff) {
    using C = Cfg<D, KC, VC>;
    ds_rd_lane<C::K_LB>(pl.k(0), a16, a8, a4, soff + C::SL_K);
    ds_rd_lane<C::K_LB>(pl.k(1), a16, a8, a4, soff + C::SL_K + C::K_TILE_BYTES);
    ds_rd_span<C::KS_LANE_BYTES>(pl.ks(0), aks, soff + C::SL_KS);
    ds_rd_span<C::KS_LANE_BYTES>(pl.ks(1), aks, soff + C::SL_KS + 32 * C::KNG);
    lds_wait<C::NWK>(pl.w);
}
// ... and the V half.
template <int D, int KC, int VC>
__device__ __forceinline__ void read_slot_v(Payload<D, KC, VC> &pl, uint32_t a16, uint32_t a8, uint32_t a4,
                                            uint32_t avs, int soff) {
    using C = Cfg<D, KC, VC>;
    ds_rd_lane<C::V_LB>(pl.v(), a16, a8, a4, soff + C::SL_V);
    ds_rd_span<C::VS_LANE_BYTES>(pl.vs(), avs, soff + C::SL_VS);
    lds_wait<C::NWV>(pl.v());
}

// Fused append, run by one wave: quantizes and stores rows [lo, hi) of kv-head
// (b, kvh) in both planes; row p comes from entry p - first of the new rows
// (app_k / app_v: [n_seqs][app_rows][n_kv_heads][D] fp32).
template <int D, int KC, int VC>
__device__ __forceinline__ void append_rows(const DecodeArgs &a, int b, int kvh, int64_t first, int64_t lo,
                                            int64_t hi, int lane) {
    constexpr int CH = D / 8;  // lanes per row (8 channels each)
    const int items = (int)(hi - lo) * CH;
    for (int it = 0; it < items; it += 64) {
        // a quantization group (G/8 lanes) never straddles rows or passes;
        // the K and V rows load together
        const int item = it + lane;
        const bool live = item < items;
        const int r = live ? item / CH : 0, chunk = item % CH;
        const int64_t pos = lo + r;
        float xk[8], xv[8];
        int64_t head_lin = 0, row = 0;
        bool ok = live;
        if (live) {
            ok = phys_row(a.k, a.pt, b, kvh, pos, head_lin, row);  // K and V pages share the table
            const int64_t off = (((int64_t)b * a.app_rows + (pos - first)) * a.k.n_kv_heads + kvh) * D + 8 * chunk;
            const float4 *pk = reinterpret_cast<const float4 *>(a.app_k + off);
            const float4 *pv = reinterpret_cast<const float4 *>(a.app_v + off);
            const float4 k0 = pk[0], k1 = pk[1], v0 = pv[0], v1 = pv[1];
            xk[0] = k0.x; xk[1] = k0.y; xk[2] = k0.z; xk[3] = k0.w;
            xk[4] = k1.x; xk[5] = k1.y; xk[6] = k1.z; xk[7] = k1.w;
            xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
            xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xk[i] = xv[i] = 0.0f;
        }
        quantize_store<KC, ROLE_K>(a.k, head_lin, row, chunk, xk, ok);
        quantize_store<VC, ROLE_V>(a.v, head_lin, row, chunk, xv, ok);
    }
}

// Splits of sequence b in this call: its rows [0, len_b) in split_rows
// pieces, at least one (an empty sequence still has its output written).
__device__ __forceinline__ int seq_splits(const DecodeArgs &a, int64_t len) {
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int64_t n = (len + a.split_rows - 1) / a.split_rows;
    return n < 1 ? 1 : (int)n;
}

// The work list of a call over several sequences: workgroup w takes the
// w-th (sequence, kv-head, split) triple, sequence-major, then kv-head, then
// split, over the splits each sequence's length needs -- so every workgroup
// with work comes before every idle one (a batch of ragged sequences sized
// by the longest leaves the idle workgroups at the end of the grid, where
// they exit at once).  The lengths stay on the device: every wave reads
// them, 64 sequences per step, and finds its triple with a prefix sum over
// the lanes; len receives the sequence's length.  False past the last
// triple.
__device__ __forceinline__ bool work_item(const DecodeArgs &a, int w, int lane, int &b, int &kvh, int &sp,
                                          int64_t &len) {
    const int H = a.k.n_kv_heads;
    int base = 0;
    for (int s0 = 0; s0 < a.n_seqs; s0 += 64) {
        const int s = s0 + lane;
        const int64_t ls = s < a.n_seqs ? a.seq_len[s] : 0;
        const int ns = s < a.n_seqs ? seq_splits(a, ls) : 0;
        const int items = ns * H;
        int incl = items;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        const int total = __shfl(incl, 63, 64);
        if (w < base + total) {
            const int r = w - base;
            const uint64_t past = __ballot(incl > r);
            const int l = __builtin_ctzll(past);
            const int first = __shfl(incl - items, l, 64);
            const int nsl = __shfl(ns, l, 64);
            b = s0 + l;
            kvh = (r - first) / nsl;
            sp = (r - first) % nsl;
            len = __shfl(ls, l, 64);
            return true;
        }
        base += total;
    }
    return false;
}

// PAGED: the planes are a page pool addressed through a.pt (else contiguous).
template <int D, int KC, int VC, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
    using C = Cfg<D, KC, VC>;
    constexpr int NS = C::NS;
    extern __shared__ __align__(16) unsigned char smem[];

    int sp, kvh, b;
    int64_t len;
    if (a.n_seqs == 1) {
        // one sequence: the grid is (kv-head, split); splits past the
        // length need no partial (the combine reads as many as it needs),
        // and the query load does not wait for the length
        b = 0;
        sp = (int)(blockIdx.x % (unsigned)a.max_splits);
        kvh = (int)(blockIdx.x / (unsigned)a.max_splits);
        len = a.seq_len[0];
        if (sp >= seq_splits(a, len)) return;  // idle: the whole workgroup
    } else {
        if (!work_item(a, blockIdx.x, threadIdx.x & 63, b, kvh, sp, len)) return;  // idle: the whole workgroup
        b = __builtin_amdgcn_readfirstlane(b);
        kvh = __builtin_amdgcn_readfirstlane(kvh);
        sp = __builtin_amdgcn_readfirstlane(sp);
        len = (int64_t)__builtin_amdgcn_readfirstlane((int)(len >> 32)) << 32 |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)len);
    }
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int64_t r0 = (int64_t)sp * a.split_rows;
    if (r0 >= len) {  // whole workgroup: no barrier reached
        if (a.max_splits > 1) {
            // the one split of an empty sequence: its partials merge as
            // nothing (max -inf, sum 0, o 0), so the combine outputs 0
            for (int i = threadIdx.x; i < a.q_len * a.gqa * D; i += kThreads) {
                const int col = i / D, qi = col / a.gqa, hh = col % a.gqa;
                const int64_t ph = (((int64_t)b * a.q_len + qi) * a.n_q_heads + (int64_t)kvh * a.gqa + hh) *
                                       a.max_splits + sp;
                a.part_o[ph * D + i % D] = 0.0f;
                if (i % D == 0) {
                    a.part_ml[2 * ph] = -INFINITY;
                    a.part_ml[2 * ph + 1] = 0.0f;
                }
            }
        } else {  // one split and an empty sequence: output 0
            for (int i = threadIdx.x; i < a.q_len * a.gqa * D; i += kThreads) {
                const int col = i / D, qi = col / a.gqa, hh = col % a.gqa;
                a.out[b * a.q_seq_stride + ((int64_t)qi * a.n_q_heads + (int64_t)kvh * a.gqa + hh) * D + i % D] = 0.0f;
            }
        }
        return;
    }
    const int nrows = (int)((r0 + a.split_rows < len) ? a.split_rows : len - r0);
    const int nblk = (nrows + kBlockRows - 1) / kBlockRows;
    const int64_t blk0 = r0 / kBlockRows;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane & 15, q4 = lane >> 4;
    const int G = a.gqa;
    const int NC = G * a.q_len;  // columns: (query, head) pairs, query-major
    // this lane's column: query qi, head hh; it sees the rows of the split
    // before nrows - cdelay (later rows are later queries' tokens)
    const int qi = h < NC ? h / G : 0, hh = h < NC ? h % G : 0;
    const int cdelay = a.q_tail + (a.q_len - 1 - qi);
    const int maxdelay = a.q_tail + a.q_len - 1;

    const int64_t head_lin = (int64_t)b * a.k.n_kv_heads + kvh;
    Streams st;
    st.kc = make_rsrc(a.k.codes + head_lin * a.k.head_code_stride + blk0 * C::K_BLOCK_BYTES,
                      (uint32_t)nblk * C::K_BLOCK_BYTES);
    st.vc = make_rsrc(a.v.codes + head_lin * a.v.head_code_stride + blk0 * C::V_BLOCK_BYTES,
                      (uint32_t)nblk * C::V_BLOCK_BYTES);
    st.ks = make_rsrc(a.k.scales + head_lin * a.k.head_scale_stride + blk0 * C::K_BLOCK_SCALES,
                      (uint32_t)nblk * C::K_BLOCK_SCALES * 2);
    st.vs = make_rsrc(a.v.scales + head_lin * a.v.head_scale_stride + blk0 * C::V_BLOCK_SCALES,
                      (uint32_t)nblk * C::V_BLOCK_SCALES * 2);
    unsigned char *myslots = smem + C::OFF_SLOTS + wave * C::NSLOT * C::SLOT;
    // paged planes: the split's page numbers, entry j in lane j % 64 of
    // pages[j / 64] (a split spans at most 128 blocks, so at most 128 pages)
    constexpr bool paged = PAGED;
    const int pblk = paged ? a.pt.page_rows / kBlockRows : 1;
    const int64_t pg0 = blk0 / pblk;
    int pages[2] = {-1, -1};
    if constexpr (paged) {
        const int64_t npg = (blk0 + nblk - 1) / pblk - pg0 + 1;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (lane + 64 * j < npg) pages[j] = a.pt.table[(int64_t)b * a.pt.table_stride + pg0 + lane + 64 * j];
    }
    // issues the DMAs of local block idx into `slot` (past the split: cut
    // off): part 0 the whole block, 1 its K half, 2 its V half
    auto issue_part = [&](int idx, unsigned char *slot, int part) {
        Streams bs = st;
        int bidx = idx;
        if constexpr (paged) {
            int page = -1, within = 0;
            if (idx < nblk) {
                const PageSlot ps = page_slot(blk0 + idx, pblk);
                const int j = (int)(ps.entry - pg0);
                page = __builtin_amdgcn_readlane(j < 64 ? pages[0] : pages[1], j & 63);
                within = ps.within;
            }
            bs = page_block_streams<D, KC, VC>(a, page, kvh, within);
            bidx = 0;
        }
        if (part == 0)
            dma_block<D, KC, VC>(bs, bidx, slot, lane);
        else
            dma_half<D, KC, VC>(bs, bidx, slot, lane, part == 1);
    };
    auto issue = [&](int idx, unsigned char *slot) { issue_part(idx, slot, 0); };

    // ---- query prologue, part 1: wave w loads the slice of channel step w
    // (8 channels per lane)
    const bool preps = wave < C::KSTEPS;
    const bool real = h < NC;
    float qv[8];
    {
        const float *qp = a.q + b * a.q_seq_stride + ((int64_t)qi * a.n_q_heads + (int64_t)kvh * G + hh) * D +
                          32 * (preps ? wave : 0) + 8 * q4;
        const float4 x0 = *reinterpret_cast<const float4 *>(qp);
        const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
        const bool use = real && preps;
        qv[0] = use ? x0.x : 0.f; qv[1] = use ? x0.y : 0.f; qv[2] = use ? x0.z : 0.f; qv[3] = use ? x0.w : 0.f;
        qv[4] = use ? x1.x : 0.f; qv[5] = use ? x1.y : 0.f; qv[6] = use ? x1.z : 0.f; qv[7] = use ? x1.w : 0.f;
    }
    // ---- fused append (app_rows > 0): wave 0 quantizes and stores this
    // split's share of the new rows [len - app_rows, len).  A DMA that could
    // read those bytes, or pull a line holding them into a cache before they
    // land (blocks from the new rows' first block minus one on; in paged
    // planes, where any block may be a memory neighbour, every block if a
    // line of scales can straddle two blocks), must not start before the
    // stores are complete.  Two ways:
    //  * flag mode (a one-block ring with a head start, the new rows in one
    //    pass of the wave, and no such block among the ones the prologue
    //    issues): wave 0 loads the new rows together with the query, stores
    //    them without waiting, and raises an LDS flag once its first
    //    complete wait (before its second block) has covered the stores; a
    //    wave that is handed such a block waits for the flag first.  Nobody
    //    else waits for the stores.
    //  * otherwise wave 0 waits for its stores before the first barrier, and
    //    such blocks are issued after that barrier.
    int dma_late = nblk;  // local blocks >= dma_late wait for the stores
    bool flag_mode = false;
    float xk[8], xv[8];
    int64_t app_hl = 0, app_row = 0;
    int app_chunk = 0;
    bool app_ok = false;
    if (a.app_rows > 0) {
        const int64_t first = len - a.app_rows;
        const int64_t lo = first > r0 ? first : r0;
        const int64_t hi = r0 + nrows;
        if (lo < hi) {
            const int nb0 = (int)((lo - r0) / kBlockRows);
            // paged: any block of the split may sit next to the new rows' one
            // in memory, which matters only where it can share a line with it
            dma_late = (paged && !C::SCALES_WHOLE_LINES) ? 0 : (nb0 > 0 ? nb0 - 1 : 0);
            constexpr int CH = D / 8;  // lanes per row (8 channels each)
            flag_mode = C::HEAD2 && dma_late >= C::NSLOT * kWaves && (hi - lo) * CH <= 64;
            if (wave == 0) {
                if (flag_mode) {
                    const int items = (int)(hi - lo) * CH;
                    const bool livei = lane < items;
                    const int r = livei ? lane / CH : 0;
                    app_chunk = lane % CH;
                    const int64_t pos = lo + r;
                    app_ok = livei && phys_row(a.k, a.pt, b, kvh, pos, app_hl, app_row);
                    if (livei) {
                        const int64_t off =
                            (((int64_t)b * a.app_rows + (pos - first)) * a.k.n_kv_heads + kvh) * D + 8 * app_chunk;
                        const float4 *pk = reinterpret_cast<const float4 *>(a.app_k + off);
                        const float4 *pv = reinterpret_cast<const float4 *>(a.app_v + off);
                        const float4 k0 = pk[0], k1 = pk[1], v0 = pv[0], v1 = pv[1];
                        xk[0] = k0.x; xk[1] = k0.y; xk[2] = k0.z; xk[3] = k0.w;
                        xk[4] = k1.x; xk[5] = k1.y; xk[6] = k1.z; xk[7] = k1.w;
                        xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w;
                        xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) xk[i] = xv[i] = 0.0f;
                    }
                } else {
                    append_rows<D, KC, VC>(a, b, kvh, first, lo, hi, lane);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
            }
        }
    }
    // the first slot starts streaming once the query is in (queued behind
    // the DMAs the query would arrive late); the rest of the ring follows the
    // prologue: a wave blocks while the memory queues are full, and the
    // prologue should not wait behind that.  The prologue touches LDS only
    // through hand-issued accesses, so it never waits for these DMAs.
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(qv[0]), "+v"(qv[1]), "+v"(qv[2]), "+v"(qv[3]), "+v"(qv[4]),
                 "+v"(qv[5]), "+v"(qv[6]), "+v"(qv[7])::"memory");
    if (flag_mode && wave == 0) {
        quantize_store<KC, ROLE_K>(a.k, app_hl, app_row, app_chunk, xk, app_ok);
        quantize_store<VC, ROLE_V>(a.v, app_hl, app_row, app_chunk, xv, app_ok);
    }
    if (wave < dma_late) issue(wave, myslots);

    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;
    if (preps) {
        float m = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) m = fmaxf(m, fabsf(qv[s]));
        m = quad_max(m);
        if (q4 == 0) ds_wr(lds0 + (wave * 16 + h) * 4, __builtin_bit_cast(uint32_t, m), C::OFF_TMAX);
    }
    if (tid == 0) {
        ds_wr(lds0, (uint32_t)(C::NSLOT * kWaves), C::OFF_CNT);
        ds_wr(lds0, 0u, C::OFF_CNT + 4);  // the new rows' stores are not known complete yet
    }
    lds_barrier();
    if (wave >= dma_late) issue(wave, myslots);

    // ---- part 2: power-of-two normalisation per head, hi + lo binary16
    // halves of channel step w, and that step's share of the bias correction
    uint32_t tmaxw[C::KSTEPS];
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) ds_rd(tmaxw[t], lds0 + h * 4, C::OFF_TMAX + t * 64);
    lds_wait<C::KSTEPS>(tmaxw);
    float qmaxabs = 0.0f;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) qmaxabs = fmaxf(qmaxabs, __builtin_bit_cast(float, tmaxw[t]));
    const int qexp = qmaxabs > 0.0f ? ilogbf(qmaxabs) : 0;
    if (preps) {
        const float qnorm = ldexpf(1.0f, -qexp);
        h8 hi8, lo8;
        float cpart = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float x = qv[s] * qnorm * k_slot_factor<KC>(s);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            hi8[s] = hi;
            lo8[s] = lo;
            cpart = fmaf((float)hi + (float)lo, k_slot_bias<KC>(s), cpart);
        }
        ds_wr(lds0 + wave * 2048 + lane * 16, __builtin_bit_cast(u4, hi8), C::OFF_QOP);
        ds_wr(lds0 + wave * 2048 + lane * 16, __builtin_bit_cast(u4, lo8), C::OFF_QOP + 1024);
        cpart = quad_sum(cpart);
        if (q4 == 0) ds_wr(lds0 + (wave * 16 + h) * 4, __builtin_bit_cast(uint32_t, cpart), C::OFF_CORR);
    }
    lds_barrier();

    uint32_t corrw[C::KSTEPS];
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) ds_rd(corrw[t], lds0 + h * 4, C::OFF_CORR + t * 64);
    lds_wait<C::KSTEPS>(corrw);
    f4 cinit[C::KNG];  // accumulator start values: cancel the operand bias
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) {
        float corr = 0.0f;
#pragma unroll
        for (int st2 = 0; st2 < C::STEPS_PER_KGROUP; ++st2)
            corr += __builtin_bit_cast(float, corrw[g * C::STEPS_PER_KGROUP + st2]);
        cinit[g] = f4{-corr, -corr, -corr, -corr};
    }
    const float c_h = a.scale_log2 * ldexpf(1.0f, qexp);
    h8 qreg[C::Q_LDS ? 1 : 2 * C::KSTEPS];
    if constexpr (!C::Q_LDS) {
#pragma unroll
        for (int i = 0; i < 2 * C::KSTEPS; ++i) ds_rd(*reinterpret_cast<u4 *>(&qreg[i]), lds0 + lane * 16, C::OFF_QOP + i * 1024);
        lds_wait<8 * C::KSTEPS>(reinterpret_cast<uint32_t *>(qreg));
    }

#pragma unroll
    for (int s = 1; s < NS; ++s) issue(wave + s * kWaves, myslots + s * C::SLOT);
    if constexpr (C::HEAD2) issue(wave + kWaves, myslots + C::SLOT);

    // LDS byte addresses for the hand-issued reads
    const uint32_t lds_slots = (uint32_t)(uintptr_t)(lds_void *)myslots;
    const uint32_t a16 = lds_slots + lane * 16, a8 = lds_slots + lane * 8, a4 = lds_slots + lane * 4;
    const uint32_t aks = lds_slots + q4 * C::KS_LANE_BYTES, avs = lds_slots + q4 * C::VS_LANE_BYTES;
    const uint32_t aq = lds0 + C::OFF_QOP + lane * 16;

    f4 O[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) O[cb] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // Computes block idx from its words.
    // rows from block idx's start to the sequence end (capped: only whether
    // it reaches past the block matters)
    auto rows_to_end = [&](int idx) -> int {
        const int64_t rte64 = len - (r0 + (int64_t)idx * kBlockRows);
        return rte64 < (1 << 20) ? (int)rte64 : (1 << 20);
    };
    // Scores, masking and the softmax update of block idx from its K half;
    // returns the probabilities (the P^T operand).
    auto process_s = [&](Payload<D, KC, VC> &pl, int idx) -> h8 {
        // ---- scores S^T for the two 16-row tiles, channel steps in lockstep
        const f16_alias *ksc0 = reinterpret_cast<const f16_alias *>(pl.ks(0));
        const f16_alias *ksc1 = reinterpret_cast<const f16_alias *>(pl.ks(1));
        float S[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int g = 0; g < C::KNG; ++g) {
            f4 acc0 = cinit[g], acc1 = cinit[g];
            h8 qg[2 * C::STEPS_PER_KGROUP];
            if constexpr (C::Q_LDS) {
#pragma unroll
                for (int i = 0; i < 2 * C::STEPS_PER_KGROUP; ++i)
                    ds_rd(*reinterpret_cast<u4 *>(&qg[i]), aq, (2 * g * C::STEPS_PER_KGROUP + i) * 1024);
                lds_wait<8 * C::STEPS_PER_KGROUP>(reinterpret_cast<uint32_t *>(qg));
            }
#pragma unroll
            for (int st2 = 0; st2 < C::STEPS_PER_KGROUP; ++st2) {
                const int t = g * C::STEPS_PER_KGROUP + st2;
                const h8 qh = C::Q_LDS ? qg[2 * st2] : qreg[2 * t];
                const h8 ql = C::Q_LDS ? qg[2 * st2 + 1] : qreg[2 * t + 1];
                const h8 k0 = k_operand<KC>(&pl.k(0)[C::K_WPS * t]);
                const h8 k1 = k_operand<KC>(&pl.k(1)[C::K_WPS * t]);
                acc0 = mfma16x16x32(k0, qh, acc0);
                acc1 = mfma16x16x32(k1, qh, acc1);
                acc0 = mfma16x16x32(k0, ql, acc0);
                acc1 = mfma16x16x32(k1, ql, acc1);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (is16(KC)) {  // binary16 keys: no scale
                    S[0][r] = acc0[r];
                    S[1][r] = acc1[r];
                } else {
                    S[0][r] = fmaf(acc0[r], (float)ksc0[g * 4 + r], S[0][r]);
                    S[1][r] = fmaf(acc1[r], (float)ksc1[g * 4 + r], S[1][r]);
                }
            }
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[tau][r] *= c_h;
        const int rend = rows_to_end(idx);
        if (rend - maxdelay < kBlockRows) {
            // row 16*tau + 4*q4 + r is visible to this column iff 16*tau + r < lim
            const int lim = rend - cdelay - 4 * q4;
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * tau + r >= lim) S[tau][r] = -INFINITY;
        }

        // ---- online softmax (log2 domain)
        float mx = S[0][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = __builtin_elementwise_maximum(mx, S[i / 4][i % 4]);
        mx = quad_max(mx);
        const bool raise = mx > m_run + kRescaleThreshold;
        if (__any(raise)) {
            const float m_new = raise ? mx : m_run;
            // 0 when raised from -inf; 1 for a lane that keeps its max (which
            // may still be -inf: a column that sees no row yet)
            const float alpha = raise ? fast_exp2(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) O[cb] *= alpha;
            m_run = m_new;
        }
        // a column that has seen no visible row yet keeps m_run = -inf; its
        // scores here are all -inf too, and exp2(-inf - 0) = 0
        const float mref = m_run > -INFINITY ? m_run : 0.0f;
        h8 P;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(S[tau][r] - mref);
                l_run += p;
                P[4 * tau + r] = (_Float16)p;
            }
        return P;
    };
    // O^T += V^T P^T for block idx from its V half.
    auto process_v = [&](Payload<D, KC, VC> &pl, int idx, const h8 &P) {
        uint32_t *vsw = pl.vs();
        const int rend = rows_to_end(idx);
        if (is16(VC) && rend < kBlockRows) {
            // binary16 values of rows past the sequence end (never written:
            // any bits) are zeroed, as the block codecs zero their scales;
            // word 4 cb + m holds the values of slots (2m, 2m + 1)
            const int vlim = rend - 4 * q4;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int j0 = (m >> 1) * 16 + 2 * (m & 1);
                    uint32_t word = pl.v()[4 * cb + m];
                    if (j0 >= vlim) word &= 0xFFFF0000u;
                    if (j0 + 1 >= vlim) word &= 0x0000FFFFu;
                    pl.v()[4 * cb + m] = word;
                }
        }
        if (!is16(VC) && rend < kBlockRows) {
            const int vlim = rend - 4 * q4;  // rows past the sequence end
            // rows past the end get a zero V scale, so that bytes that were
            // never written cannot turn 0 * V into NaN; word g*4+m holds the
            // scales of rows (m/2)*16 + 4*q4 + 2*(m%2) + {0, 1}
#pragma unroll
            for (int g = 0; g < C::VNG; ++g)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int j0 = (m >> 1) * 16 + 2 * (m & 1);
                    uint32_t word = vsw[g * 4 + m];
                    if (j0 >= vlim) word &= 0xFFFF0000u;
                    if (j0 + 1 >= vlim) word &= 0x0000FFFFu;
                    vsw[g * 4 + m] = word;
                }
        }
        const h2_alias *svb = reinterpret_cast<const h2_alias *>(vsw);

        // ---- O^T += V^T P^T, one 16-channel block at a time
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const int gv = is16(VC) ? 0 : cb * 16 / C::VG;
            const h8 vop = v_operand<VC>(&pl.v()[C::V_WPC * cb], svb + gv * 4);
            O[cb] = mfma16x16x32(vop, P, O[cb]);
        }
    };
    auto process = [&](Payload<D, KC, VC> &pl, int idx) {
        const h8 P = process_s(pl, idx);
        process_v(pl, idx, P);
    };

    // ---- the ring.  Slot s starts with block w + 8 s; each refill takes the
    // next unclaimed block of the split from the workgroup's LDS counter, so
    // waves whose blocks arrive early take more of them.  A wave's slots hold
    // increasing block indices, so the first one past the end ends the wave.
    // At the top of a slot the DMAs issued after its own are those of the
    // NS - 1 other slots: waiting until at most that many remain is exact.
    // Waits until wave 0 has raised the flag (its stores of the new rows are
    // complete).  Wave 0 raises it without waiting for any other wave, so the
    // wait ends; the poll count only bounds it (a.append_wait_polls).  A wait
    // that runs out goes on, so the kernel always ends, and reports it: the
    // block it then reads may hold the new rows' old bytes.
    auto wait_appended = [&]() {
        for (int it = 0; it < a.append_wait_polls; ++it) {
            uint32_t f;
            ds_rd(f, lds0, C::OFF_CNT + 4);
            lds_wait<1>(&f);
            if (__builtin_amdgcn_readfirstlane(f) != 0u) return;
            __builtin_amdgcn_s_sleep(2);
        }
        if (a.dev_status && lane == 0) *a.dev_status = kStatusWaitExpired;
    };
    auto grab = [&]() -> int {
        uint32_t v = 0;
        if (lane == 0) v = ds_add_rtn(lds0, 1u, C::OFF_CNT);
        return __builtin_amdgcn_readfirstlane((int)v);
    };
    int sidx[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) sidx[s] = wave + s * kWaves;
    if constexpr (C::HEAD2) {
        // slot 0 holds block `wave`, slot 1 block `wave + 8`: the first is
        // consumed without a refill, the second refills slot 0, where the
        // one-block ring then continues
        if (wave < nblk) {
            vm_wait<C::N_DMA>();
            Payload<D, KC, VC> pl;
            read_slot<D, KC, VC>(pl, a16, a8, a4, aks, avs, 0);
            process(pl, wave);
        }
        sidx[0] = nblk;
        if (wave + kWaves < nblk) {
            vm_wait<0>();
            // in flag mode wave 0 always gets here (its second block exists),
            // and this complete wait covered its stores of the new rows
            if (flag_mode && wave == 0 && !a.hold_append_flag) ds_wr(lds0, 1u, C::OFF_CNT + 4);
            Payload<D, KC, VC> pl;
            read_slot<D, KC, VC>(pl, a16, a8, a4, aks, avs, C::SLOT);
            const int nxt = grab();
            sidx[0] = nxt;
            if (flag_mode && nxt >= dma_late && nxt < nblk) wait_appended();
            issue(nxt, myslots);
            process(pl, wave + kWaves);
        }
    }
    if constexpr (C::TWO_PHASE) {
        // one slot, refilled half by half: the K half of the next block is
        // requested once this block's K half is copied, its V half once this
        // block's V half is copied.  DMA order K(n), V(n), K(n+1), V(n+1):
        // K(n) has landed when at most the V(n) DMAs remain, V(n) when at
        // most the K(n+1) DMAs remain.
        int cur = wave;
        while (cur < nblk) {
            Payload<D, KC, VC> pl;
            vm_wait<C::N_DMA_V>();
            read_slot_k<D, KC, VC>(pl, a16, a8, a4, aks, 0);
            const int nxt = grab();
            issue_part(nxt, myslots, 1);
            const h8 P = process_s(pl, cur);
            vm_wait<C::N_DMA_K>();
            read_slot_v<D, KC, VC>(pl, a16, a8, a4, avs, 0);
            issue_part(nxt, myslots, 2);
            process_v(pl, cur, P);
            cur = nxt;
        }
        sidx[0] = nblk;  // the ring below has nothing left
    }
    bool live = true;
    while (live) {
        [&]<int... S>(std::integer_sequence<int, S...>) {
            (([&] {
                 if (!live) return;
                 const int idx = sidx[S];
                 if (idx >= nblk) { live = false; return; }
                 vm_wait<(NS - 1) * C::N_DMA>();
                 Payload<D, KC, VC> pl;
                 read_slot<D, KC, VC>(pl, a16, a8, a4, aks, avs, S * C::SLOT);
                 const int nxt = grab();
                 sidx[S] = nxt;
                 if (flag_mode && nxt >= dma_late && nxt < nblk) wait_appended();
                 issue(nxt, myslots + S * C::SLOT);
                 process(pl, idx);
             }()),
             ...);
        }(std::make_integer_sequence<int, NS>{});
    }

    // ---- merge the waves.
    l_run = quad_sum(l_run);
    constexpr int D4 = D / 4;
    // writes item (col, c) of the merged result: the output when the call has
    // one split, else this split's partial (unnormalized O, max, sum).  A
    // V_hat beyond the binary16 range (|code * dq| > 65504) became an
    // infinity in the operand, which reaches the sums it enters as an
    // infinity or a NaN (0 * inf included); a non-finite item marks the call
    // as outside the operand range (finite queries assumed), and the
    // combine of finite partials stays finite.
    auto emit = [&](int col, int c, const f4 &o, float M, float L) {
        if (a.dev_status && !(__builtin_isfinite(o[0]) && __builtin_isfinite(o[1]) && __builtin_isfinite(o[2]) &&
                              __builtin_isfinite(o[3])))
            *a.dev_status = kStatusOverflow;
        const int cq = col / G, ch = col % G;
        if (a.max_splits == 1) {
            const float r = L > 0.0f ? 1.0f / L : 0.0f;
            float *dst = a.out + b * a.q_seq_stride + ((int64_t)cq * a.n_q_heads + (int64_t)kvh * G + ch) * D + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = o[i] * r;
            return;
        }
        const int64_t qh = ((int64_t)b * a.q_len + cq) * a.n_q_heads + (int64_t)kvh * G + ch;
        const int64_t ph = qh * a.max_splits + sp;
        *reinterpret_cast<f4 *>(a.part_o + ph * D + c) = o;
        if (c == 0) {
            a.part_ml[2 * ph] = M;
            a.part_ml[2 * ph + 1] = L;
        }
    };
    if (NC * C::DP * 4 <= C::NSLOT * C::SLOT) {
        // Each wave parks its unscaled O and its (max, sum) as soon as its
        // own blocks are done -- in its own slots, which no other wave
        // touches -- so the parking overlaps the waves still streaming; after
        // one barrier each thread weighs the 8 copies of 4 channels of one
        // column by 2^(max_w - max).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's last DMAs have landed
        float *mm = reinterpret_cast<float *>(smem + C::OFF_ML);  // [16][wave] max, then [16][wave] sum
        if (h < NC) {
            float *own = reinterpret_cast<float *>(myslots) + h * C::DP + 4 * q4;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) *reinterpret_cast<f4 *>(own + 16 * cb) = O[cb];
            if (q4 == 0) {
                mm[h * kWaves + wave] = m_run;
                mm[16 * kWaves + h * kWaves + wave] = l_run;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < NC * D4; idx += kThreads) {
            const int col = idx / D4, c = (idx % D4) * 4;
            float mw[kWaves], lw[kWaves];
#pragma unroll
            for (int w = 0; w < kWaves; w += 4) {
                const f4 x = *reinterpret_cast<const f4 *>(mm + col * kWaves + w);
                const f4 y = *reinterpret_cast<const f4 *>(mm + 16 * kWaves + col * kWaves + w);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mw[w + i] = x[i];
                    lw[w + i] = y[i];
                }
            }
            float M = mw[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
            const float Mref = M > -INFINITY ? M : 0.0f;  // -inf: no visible row in the split
            float L = 0.0f;
            f4 o = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float e = fast_exp2(mw[w] - Mref);  // 0 for a wave without visible rows
                L = fmaf(e, lw[w], L);
                const f4 x = *reinterpret_cast<const f4 *>(
                    reinterpret_cast<const float *>(smem + C::OFF_SLOTS + w * C::NSLOT * C::SLOT) + col * C::DP + c);
                o = f4{fmaf(e, x[0], o[0]), fmaf(e, x[1], o[1]), fmaf(e, x[2], o[2]), fmaf(e, x[3], o[3])};
            }
            emit(col, c, o, M, L);
        }
        return;
    }
    // Otherwise each wave publishes its (max, sum) per column; after one
    // barrier (which also waited for every wave's last DMAs, so the slots are
    // idle) every wave rescales its O to the columns' common max and parks it
    // in the slot area; after a second barrier the threads add up the 8
    // parked copies, 4 channels each.
    float *sml = reinterpret_cast<float *>(smem + C::OFF_ML);    // [wave][16][2]
    float *sfin = reinterpret_cast<float *>(smem + C::OFF_FIN);  // [16][2]
    if (h < NC && q4 == 0) {
        sml[(wave * 16 + h) * 2] = m_run;
        sml[(wave * 16 + h) * 2 + 1] = l_run;
    }
    __syncthreads();
    if (h < NC) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sml[(w * 16 + h) * 2]);
        const float Mref = M > -INFINITY ? M : 0.0f;  // -inf: no visible row in the split
        const float e = fast_exp2(m_run - Mref);      // 0 for a wave without visible rows
        float *own = reinterpret_cast<float *>(smem + C::OFF_SLOTS) + (wave * NC + h) * C::DP + 4 * q4;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const f4 x = O[cb];
            *reinterpret_cast<f4 *>(own + 16 * cb) = f4{x[0] * e, x[1] * e, x[2] * e, x[3] * e};
        }
        if (wave == 0 && q4 == 0) {
            float L = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                L = fmaf(fast_exp2(sml[(w * 16 + h) * 2] - Mref), sml[(w * 16 + h) * 2 + 1], L);
            sfin[2 * h] = M;
            sfin[2 * h + 1] = L;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < NC * D4; idx += kThreads) {
        const int col = idx / D4, c = (idx % D4) * 4;
        const float *src = reinterpret_cast<const float *>(smem + C::OFF_SLOTS) + col * C::DP + c;
        f4 o = *reinterpret_cast<const f4 *>(src);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const f4 x = *reinterpret_cast<const f4 *>(src + w * NC * C::DP);
            o = f4{o[0] + x[0], o[1] + x[1], o[2] + x[2], o[3] + x[3]};
        }
        emit(col, c, o, sfin[2 * col], sfin[2 * col + 1]);
    }
}

// Log-sum-exp merge of the splits of one (sequence, query, head), 64 channels
// per workgroup: 4 thread groups take every 4th split; each thread issues the
// loads of 16 splits at once and folds them into a running (max, sum, output)
// triple, then the 4 groups merge through LDS.  The sequence's splits (as
// many as its length needs, see seq_splits) each have a partial (an empty or
// invisible one carries max -inf, sum 0, o 0); a query that sees no row at
// all gets 0.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
    __shared__ float s_o[4][64], s_m[4][64], s_l[4][64];
    const int hq = blockIdx.y, row = blockIdx.z, tid = threadIdx.x;
    const int b = row / a.q_len, qi = row % a.q_len;
    const int nsp = seq_splits(a, a.seq_len[b]);
    const int64_t qh = (int64_t)row * a.n_q_heads + hq;
    const int cl = tid & 63, sg = tid >> 6, c = blockIdx.x * 64 + cl;
    const float *ml = a.part_ml + 2 * qh * a.max_splits;
    const float *po = a.part_o + qh * a.max_splits * D + c;
    constexpr int U = 16;
    float M = -INFINITY, o = 0.0f, L = 0.0f;
    for (int s0 = sg; s0 < nsp; s0 += 4 * U) {
        float mv[U], lv[U], ov[U];
        // every load is issued (a split past the end re-reads the last one),
        // so all of them are in flight together behind a single wait; the
        // surplus values are dropped afterwards
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s2 = s0 + 4 * u < nsp ? s0 + 4 * u : nsp - 1;
            const float2 x = *reinterpret_cast<const float2 *>(ml + 2 * s2);
            mv[u] = x.x;
            lv[u] = x.y;
            ov[u] = po[(int64_t)s2 * D];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = s0 + 4 * u < nsp;
            mv[u] = ok ? mv[u] : -INFINITY;
            lv[u] = ok ? lv[u] : 0.0f;
            ov[u] = ok ? ov[u] : 0.0f;
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < U; ++u) mb = fmaxf(mb, mv[u]);
        const float mref = mb > -INFINITY ? mb : 0.0f;     // all -inf so far: nothing to scale
        const float sc = fast_exp2(M - mref);              // 0 on the first chunk
        o *= sc;
        L *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float e = fast_exp2(mv[u] - mref);
            o = fmaf(e, ov[u], o);
            L = fmaf(e, lv[u], L);
        }
        M = mb;
    }
    s_o[sg][cl] = o;
    s_m[sg][cl] = M;
    s_l[sg][cl] = L;
    __syncthreads();
    if (sg == 0) {
        float Mt = s_m[0][cl];
#pragma unroll
        for (int g = 1; g < 4; ++g) Mt = fmaxf(Mt, s_m[g][cl]);
        const float Mref = Mt > -INFINITY ? Mt : 0.0f;
        float on = 0.0f, Ln = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float e = fast_exp2(s_m[g][cl] - Mref);  // 0 for a group without splits
            on = fmaf(e, s_o[g][cl], on);
            Ln = fmaf(e, s_l[g][cl], Ln);
        }
        a.out[b * a.q_seq_stride + ((int64_t)qi * a.n_q_heads + hq) * D + c] = Ln > 0.0f ? on / Ln : 0.0f;
    }
}

template <int D, int KC, int VC>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
    using C = Cfg<D, KC, VC>;
    const size_t merge_lds = (size_t)C::OFF_SLOTS + (size_t)kWaves * a.gqa * a.q_len * C::DP * sizeof(float);
    const size_t lds = (size_t)C::LDS_STREAM > merge_lds ? (size_t)C::LDS_STREAM : merge_lds;
    // one workgroup per (sequence, kv-head, split) the longest sequence would
    // need; those past the work list (shorter sequences) exit at once
    const dim3 grid((unsigned)((int64_t)a.max_splits * a.k.n_kv_heads * a.n_seqs));
    const void *fn = a.pt.table ? (const void *)decode_kernel<D, KC, VC, true>
                                : (const void *)decode_kernel<D, KC, VC, false>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (a.pt.table)
        decode_kernel<D, KC, VC, true><<<grid, dim3(kThreads), lds, s>>>(a);
    else
        decode_kernel<D, KC, VC, false><<<grid, dim3(kThreads), lds, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_splits <= 1) return e;
    combine_kernel<D><<<dim3(D / 64, (unsigned)a.n_q_heads, (unsigned)(a.n_seqs * a.q_len)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    switch (a.k.codec * 3 + a.v.codec) {
        case Q8_0 * 3 + Q8_0: return launch_typed<D, Q8_0, Q8_0>(a, s);
        case Q8_0 * 3 + Q4_0: return launch_typed<D, Q8_0, Q4_0>(a, s);
        case Q8_0 * 3 + Q4_G64: return launch_typed<D, Q8_0, Q4_G64>(a, s);
        case Q4_0 * 3 + Q8_0: return launch_typed<D, Q4_0, Q8_0>(a, s);
        case Q4_0 * 3 + Q4_0: return launch_typed<D, Q4_0, Q4_0>(a, s);
        case Q4_0 * 3 + Q4_G64: return launch_typed<D, Q4_0, Q4_G64>(a, s);
        case Q4_G64 * 3 + Q8_0: return launch_typed<D, Q4_G64, Q8_0>(a, s);
        case Q4_G64 * 3 + Q4_0: return launch_typed<D, Q4_G64, Q4_0>(a, s);
        case Q4_G64 * 3 + Q4_G64: return launch_typed<D, Q4_G64, Q4_G64>(a, s);
        case F16 * 3 + F16:
            if constexpr (D <= 128) return launch_typed<D, F16, F16>(a, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

DecodePlan plan_decode(int head_dim, int n_kv_heads, int n_q_heads, int n_seqs, int64_t max_len,
                       int q_len) {
    // Enough rows per workgroup that the partials stay small next to the KV
    // bytes, few enough that ~one workgroup per compute unit (256) is busy;
    // long multi-sequence calls get more, shorter splits for load balance.
    const int64_t blocks_per_head = (max_len + kBlockRows - 1) / kBlockRows;
    const int64_t total_blocks = blocks_per_head * n_kv_heads * (int64_t)n_seqs;
    int64_t per_split = (total_blocks + 255) / 256;
    if (per_split < kWaves) per_split = kWaves;
    if (per_split > 128) per_split = 128;
    per_split = (per_split + kWaves - 1) / kWaves * kWaves;
    DecodePlan p;
    p.split_rows = (int)(per_split * kBlockRows);
    p.max_splits = (int)((max_len + p.split_rows - 1) / p.split_rows);
    if (p.max_splits < 1) p.max_splits = 1;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    p.part_ml_bytes = (size_t)n_seqs * q_len * n_q_heads * p.max_splits * 2 * sizeof(float);
    p.part_o_bytes = (size_t)n_seqs * q_len * n_q_heads * p.max_splits * head_dim * sizeof(float);
    p.off_part_ml = 0;
    p.off_part_o = p.off_part_ml + up(p.part_ml_bytes);
    p.total_bytes = p.off_part_o + up(p.part_o_bytes);
    return p;
}

// ---- the no-allocation entry point's scratch ----------------------------------
// Split partials of kvq_append_attend_decode_noalloc.  In host code the
// array's name stands for a host-side handle, not a device address: only the
// address hipGetSymbolAddress returns (per GPU, with that GPU current) is
// ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(hipStream_t s, void **ptr) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (e2 != hipSuccess) return e2;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool decode_supported(int k_codec, int v_codec, int head_dim) {
    if (k_codec == F16 || v_codec == F16)  // the f16 control: f16/f16 at head_dim 64 and 128
        return k_codec == F16 && v_codec == F16 && (head_dim == 64 || head_dim == 128);
    return k_codec >= 0 && k_codec <= 2 && v_codec >= 0 && v_codec <= 2 &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    switch (a.k.head_dim) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
