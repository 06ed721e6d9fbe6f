// attn_decode.hip -- split-K decode attention over the block-quantized cache,
// plus the log-sum-exp combine of the splits.  gfx950.
//
// What is computed (den_llama.cpp, "Results" / "What's in the fork":
// FlashAttention reads the q8_0 / q4_0 / Q4_G64 K and V blocks directly):
//   out[b][h] = sum_j softmax_j(scale * q[b][h] . k_hat_j) v_hat_j over the
//   rows j < len_b of kv-head h / gqa.
//
// Design (one workgroup = 8 waves = one split of `split_rows` rows of one
// (sequence, kv-head); each wave takes every 8th 32-row block of the split):
//  * The GQA group (<= 16 query heads) is the N side of 16x16x32 f16 matrix
//    products, so every K/V byte is read once per kv-head:
//      S^T[row][head] = K[row][:] . Q'[:][head]   (A = K codes, B = query)
//      O^T[ch][head] += V[ch][rows] . P^T[rows][head]
//    The accumulator layout of S^T (lane = head + 16*q holds rows 4q..4q+3 of
//    each 16-row tile) is exactly the B-operand layout P^T needs, and the
//    V-role block layout puts each lane's eight V rows where its probabilities
//    are, so no data moves between the two products.
//  * K codes enter the matrix cores as exact binary16 "1024 + n" / "1152 + b"
//    values (two masks, a shift or a byte permute per word); the constant
//    bias is cancelled by starting the accumulator at -sum(query * bias).
//    The query is scaled by a power of two and split into hi + lo binary16
//    halves (two products), so the score keeps ~22 bits.  K group scales are
//    applied in fp32 to each group's partial dot product.
//  * V enters as binary16 code * dq (one rounding, exact for subnormal dq);
//    probabilities enter as binary16.  Statistics and sums are fp32.
//  * Online softmax in log2 units; the running max is only raised when a
//    block exceeds it by more than 8 (probabilities stay <= 256), so the
//    64-register rescale of O is rare.
//  * Each wave prefetches its next 32-row block (code words and a slice of
//    the block's scales) into registers while it computes the current one;
//    the scales go through a per-wave LDS slot to reach operand order.
//    Blocks are handed out dynamically inside the workgroup (LDS counter), so
//    the 8 waves finish together.
//  * The workgroup's query rows are staged once in LDS (coalesced), so the
//    many workgroups of one kv-head do not all hammer the same few lines.
//  * The 8 waves merge through LDS; each workgroup writes one partial
//    (unnormalized O, max, sum) per query head, or the final output when the
//    sequence fits in one split; combine_kernel merges the splits
//    (log-sum-exp) with many partial loads in flight at once.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleThreshold = 8.0f;

template <int D, int KC, int VC>
struct Cfg {
    static constexpr int KSTEPS = D / 32;
    static constexpr int KG = group_size(KC);
    static constexpr int KNG = D / KG;
    static constexpr int STEPS_PER_KGROUP = KG / 32;
    static constexpr int VG = group_size(VC);
    static constexpr int VNG = D / VG;
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
    static constexpr int KS_WORDS = K_BLOCK_SCALES / 2;  // 32-bit words of K scales per block
    static constexpr int VS_WORDS = V_BLOCK_SCALES / 2;
    static constexpr int KS_PER_LANE = (KS_WORDS + 63) / 64;
    static constexpr int VS_PER_LANE = (VS_WORDS + 63) / 64;
    // head_dim 256: the query's low half lives in a per-wave LDS copy (read
    // once per k-step) to leave registers for two blocks in flight
    static constexpr bool QLO_LDS = D == 256;
    static constexpr int SLOT_WORDS = KS_WORDS + VS_WORDS;
    static constexpr int QLO_BYTES = QLO_LDS ? KSTEPS * 64 * 16 : 0;  // per wave
    static constexpr int QOFF = kWaves * (SLOT_WORDS * 4 + QLO_BYTES);  // staged query rows
};

// Loads the LB bytes lane `lane` owns in a chunk-major region into words.
template <int LB>
__device__ __forceinline__ void load_lane_words(const uint8_t *region, int lane, uint32_t *w) {
    constexpr int W = chunk_width(LB);
    if constexpr (W == 16) {
#pragma unroll
        for (int c = 0; c < LB / 16; ++c) {
            const u4 v = *reinterpret_cast<const u4 *>(region + c * 1024 + lane * 16);
            w[4 * c + 0] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
        }
    } else if constexpr (W == 8) {
        const u2 v = *reinterpret_cast<const u2 *>(region + lane * 8);
        w[0] = v.x; w[1] = v.y;
    } else {
        static_assert(W == 4, "lane chunk width");
        w[0] = *reinterpret_cast<const uint32_t *>(region + lane * 4);
    }
}

// Everything one wave needs from HBM for one 32-row block: its K and V code
// words and one slice of the block's K and V scales (the whole wave loads each
// block's scales with one coalesced pass, then stages them in its own LDS slot
// to read them back in operand order).
template <int D, int KC, int VC>
struct Buf {
    using C = Cfg<D, KC, VC>;
    uint32_t k[2][C::K_WORDS];
    uint32_t v[C::V_WORDS];
    uint32_t ks[C::KS_PER_LANE];
    uint32_t vs[C::VS_PER_LANE];
};

template <int D, int KC, int VC>
__device__ __forceinline__ void load_buf(Buf<D, KC, VC> &bf, const uint8_t *kblk, const uint8_t *vblk,
                                         const uint32_t *ksb, const uint32_t *vsb, int lane) {
    using C = Cfg<D, KC, VC>;
    load_lane_words<C::K_LB>(kblk, lane, bf.k[0]);
    load_lane_words<C::K_LB>(kblk + C::K_TILE_BYTES, lane, bf.k[1]);
    load_lane_words<C::V_LB>(vblk, lane, bf.v);
#pragma unroll
    for (int i = 0; i < C::KS_PER_LANE; ++i) {
        const int w = lane + 64 * i;
        bf.ks[i] = w < C::KS_WORDS ? ksb[w] : 0u;
    }
#pragma unroll
    for (int i = 0; i < C::VS_PER_LANE; ++i) {
        const int w = lane + 64 * i;
        bf.vs[i] = w < C::VS_WORDS ? vsb[w] : 0u;
    }
}

template <int D, int KC, int VC>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
    using C = Cfg<D, KC, VC>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_next;

    const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    int64_t len = a.seq_len[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int64_t r0 = (int64_t)sp * a.split_rows;
    if (r0 >= len) {  // whole workgroup: no barrier reached
        if (len == 0 && sp == 0) {  // an empty sequence attends nothing: output 0
            float *dst = a.out + ((int64_t)b * a.n_q_heads + (int64_t)kvh * a.gqa) * D;
            for (int i = threadIdx.x; i < a.gqa * D; i += kThreads) dst[i] = 0.0f;
        }
        return;
    }
    const int nrows = (int)((r0 + a.split_rows < len) ? a.split_rows : len - r0);
    const int nblk = (nrows + kBlockRows - 1) / kBlockRows;
    const int64_t blk0 = r0 / kBlockRows;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane & 15, q4 = lane >> 4;
    const int G = a.gqa;

    const int64_t head_lin = (int64_t)b * a.k.n_kv_heads + kvh;
    const uint8_t *kcodes = a.k.codes + head_lin * a.k.head_code_stride + blk0 * C::K_BLOCK_BYTES;
    const uint8_t *vcodes = a.v.codes + head_lin * a.v.head_code_stride + blk0 * C::V_BLOCK_BYTES;
    const uint32_t *kscales = reinterpret_cast<const uint32_t *>(
        a.k.scales + head_lin * a.k.head_scale_stride + blk0 * C::K_BLOCK_SCALES);
    const uint32_t *vscales = reinterpret_cast<const uint32_t *>(
        a.v.scales + head_lin * a.v.head_scale_stride + blk0 * C::V_BLOCK_SCALES);
    auto issue = [&](Buf<D, KC, VC> &bf, int idx) {
        load_buf<D, KC, VC>(bf, kcodes + (int64_t)idx * C::K_BLOCK_BYTES,
                            vcodes + (int64_t)idx * C::V_BLOCK_BYTES,
                            kscales + (int64_t)idx * C::KS_WORDS, vscales + (int64_t)idx * C::VS_WORDS,
                            lane);
    };

    // ---- the workgroup's G query rows (G*D fp32, contiguous) go to LDS once
    // with coalesced loads; each wave then reads its operand slice from there.
    float *sq = reinterpret_cast<float *>(smem + C::QOFF);
    {
        const float4 *qsrc = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)b * a.n_q_heads + (int64_t)kvh * G) * D);
        for (int i = tid; i < G * D / 4; i += kThreads) reinterpret_cast<float4 *>(sq)[i] = qsrc[i];
    }
    // ---- blocks are handed out dynamically inside the workgroup: wave w
    // starts with block w, then each wave takes the next unclaimed block.
    if (tid == 0) s_next = kWaves;
    Buf<D, KC, VC> bufA, bufB;
    int cur = wave;
    if (cur < nblk) issue(bufA, cur);
    __syncthreads();  // s_next initialised, query staged
    float qv[C::KSTEPS][8];
    {
        const bool real = h < G;
        const float *qp = sq + (real ? h : 0) * D;
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
            const float4 x0 = *reinterpret_cast<const float4 *>(qp + 32 * t + 8 * q4);
            const float4 x1 = *reinterpret_cast<const float4 *>(qp + 32 * t + 8 * q4 + 4);
            qv[t][0] = real ? x0.x : 0.f; qv[t][1] = real ? x0.y : 0.f;
            qv[t][2] = real ? x0.z : 0.f; qv[t][3] = real ? x0.w : 0.f;
            qv[t][4] = real ? x1.x : 0.f; qv[t][5] = real ? x1.y : 0.f;
            qv[t][6] = real ? x1.z : 0.f; qv[t][7] = real ? x1.w : 0.f;
        }
    }
    auto grab = [&]() -> int {
        int v = 0;
        if (lane == 0) v = atomicAdd(&s_next, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };
    int nxt = cur < nblk ? grab() : nblk;
    if (nxt < nblk) issue(bufB, nxt);

    // ---- query operand: power-of-two normalised hi + lo binary16 halves
    float qmaxabs = 0.0f;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s) qmaxabs = fmaxf(qmaxabs, fabsf(qv[t][s]));
    qmaxabs = fmaxf(qmaxabs, shfl_xor(qmaxabs, 16));
    qmaxabs = fmaxf(qmaxabs, shfl_xor(qmaxabs, 32));
    const int qexp = qmaxabs > 0.0f ? ilogbf(qmaxabs) : 0;
    const float qnorm = ldexpf(1.0f, -qexp);
    h8 qhi[C::KSTEPS], qlo[C::QLO_LDS ? 1 : C::KSTEPS];
    h8 *qlo_lds = reinterpret_cast<h8 *>(smem + kWaves * C::SLOT_WORDS * 4) +
                  (size_t)wave * C::KSTEPS * 64 + lane;
    float corr[C::KNG];
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) corr[g] = 0.0f;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) {
        float cpart = 0.0f;  // exact: at most 8 products of 11-bit values and a 5-bit bias
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float x = qv[t][s] * qnorm * k_slot_factor<KC>(s);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            qhi[t][s] = hi;
            qlo[C::QLO_LDS ? 0 : t][s] = lo;
            cpart = fmaf((float)hi + (float)lo, k_slot_bias<KC>(s), cpart);
        }
        if constexpr (C::QLO_LDS) qlo_lds[t * 64] = qlo[0];
        corr[t / C::STEPS_PER_KGROUP] += cpart;
    }
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) {
        corr[g] += shfl_xor(corr[g], 16);
        corr[g] += shfl_xor(corr[g], 32);
    }
    const float c_h = a.scale_log2 * ldexpf(1.0f, qexp);
    f4 cinit[C::KNG];  // accumulator start values: cancel the operand bias
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) cinit[g] = f4{-corr[g], -corr[g], -corr[g], -corr[g]};

    // per-wave LDS slot for one block's scales
    uint32_t *slot = reinterpret_cast<uint32_t *>(smem) + wave * C::SLOT_WORDS;

    f4 O[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) O[cb] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    auto process = [&](const Buf<D, KC, VC> &bf, int idx) {
        // stage this block's scales, read them back in operand order
        const int rows_here = nrows - idx * kBlockRows;  // > 0
#pragma unroll
        for (int i = 0; i < C::KS_PER_LANE; ++i)
            if (lane + 64 * i < C::KS_WORDS) slot[lane + 64 * i] = bf.ks[i];
#pragma unroll
        for (int i = 0; i < C::VS_PER_LANE; ++i) {
            const int w = lane + 64 * i;
            if (w < C::VS_WORDS) {
                uint32_t word = bf.vs[i];
                if (rows_here < kBlockRows) {
                    // rows past the end get a zero V scale, so that bytes that
                    // were never written cannot turn 0 * V into NaN
                    const int m = w & 3;
                    const int j0 = (m >> 1) * 16 + 4 * (w / (4 * C::VNG)) + 2 * (m & 1);
                    if (j0 >= rows_here) word &= 0xFFFF0000u;
                    if (j0 + 1 >= rows_here) word &= 0x0000FFFFu;
                }
                slot[C::KS_WORDS + w] = word;
            }
        }
        // ---- scores S^T for the two 16-row tiles
        float S[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const _Float16 *ksc = reinterpret_cast<const _Float16 *>(slot) + tau * 16 * C::KNG +
                                  q4 * 4 * C::KNG;
            float sacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < C::KNG; ++g) {
                f4 acc = cinit[g];
#pragma unroll
                for (int st = 0; st < C::STEPS_PER_KGROUP; ++st) {
                    const int t = g * C::STEPS_PER_KGROUP + st;
                    const h8 kop = k_operand<KC>(&bf.k[tau][is8(KC) ? 2 * t : t]);
                    acc = mfma16x16x32(kop, qhi[t], acc);
                    if constexpr (C::QLO_LDS) acc = mfma16x16x32(kop, qlo_lds[t * 64], acc);
                    else acc = mfma16x16x32(kop, qlo[t], acc);
                }
                if (C::KNG >= 4 && (g & 1) == 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[r] = fmaf(acc[r], (float)ksc[g * 4 + r], sacc[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) S[tau][r] = sacc[r] * c_h;
            __builtin_amdgcn_sched_barrier(0);  // keep one tile's operands live at a time
        }
        if (rows_here < kBlockRows) {
            const int lim = rows_here - 4 * q4;  // row 16*tau + 4*q4 + r is valid iff 16*tau + r < lim
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * tau + r >= lim) S[tau][r] = -INFINITY;
        }
        const h2 *svb = reinterpret_cast<const h2 *>(slot + C::KS_WORDS) + q4 * 4 * C::VNG;

        // ---- online softmax (log2 domain)
        float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                         fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const bool raise = mx > m_run + kRescaleThreshold;
        if (__any(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = fast_exp2(m_run - m_new);  // 0 on the first block
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) O[cb] *= alpha;
            m_run = m_new;
        }
        h8 P;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = fast_exp2(S[tau][r] - m_run);
                l_run += p;
                P[4 * tau + r] = (_Float16)p;
            }

        __builtin_amdgcn_sched_barrier(0);
        // ---- O^T += V^T P^T, one 16-channel block at a time
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const int gv = cb * 16 / C::VG;
            const h8 vop = v_operand<VC>(&bf.v[is8(VC) ? 2 * cb : cb], svb + gv * 4);
            O[cb] = mfma16x16x32(vop, P, O[cb]);
            if ((cb & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the unpacked operands in flight
        }
    };

    while (cur < nblk) {
        process(bufA, cur);
        cur = nxt;
        if (cur >= nblk) break;
        bufA = bufB;  // register renames after full unrolling of the copy
        nxt = grab();
        if (nxt < nblk) issue(bufB, nxt);
    }

    // ---- merge the 8 waves through LDS
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    __syncthreads();
    constexpr int DP = D + 4;                               // padded head stride
    float *so = reinterpret_cast<float *>(smem);           // [wave][G][DP]
    float *sm = so + kWaves * G * DP;                       // [wave][G]
    float *sl = sm + kWaves * G;                            // [wave][G]
    if (h < G) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
            *reinterpret_cast<f4 *>(&so[(wave * G + h) * DP + 16 * cb + 4 * q4]) = O[cb];
        if (q4 == 0) {
            sm[wave * G + h] = m_run;
            sl[wave * G + h] = l_run;
        }
    }
    __syncthreads();
    const int nsp = (int)((len + a.split_rows - 1) / a.split_rows);
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int hh = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * G + hh]);
        float o = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = fast_exp2(sm[w * G + hh] - M);  // 0 for waves without rows
            o = fmaf(e, so[(w * G + hh) * DP + c], o);
            L = fmaf(e, sl[w * G + hh], L);
        }
        const int64_t qh = (int64_t)b * a.n_q_heads + (int64_t)kvh * G + hh;
        if (nsp == 1) {
            a.out[qh * D + c] = o / L;
            continue;
        }
        const int64_t ph = qh * a.max_splits + sp;
        a.part_o[ph * D + c] = o;
        if (c == 0) {
            a.part_ml[2 * ph] = M;
            a.part_ml[2 * ph + 1] = L;
        }
    }
}

// Log-sum-exp merge of the splits of one (sequence, query head), 64 channels
// per workgroup: 4 thread groups take every 4th split; each thread issues the
// loads of 16 splits at once and folds them into a running (max, sum, output)
// triple, then the 4 groups merge through LDS.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
    __shared__ float s_o[4][64], s_m[4][64], s_l[4][64];
    const int hq = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    int64_t len = a.seq_len[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int nsp = (int)((len + a.split_rows - 1) / a.split_rows);
    if (nsp <= 1) return;  // the decode kernel wrote the output itself
    const int64_t qh = (int64_t)b * a.n_q_heads + hq;
    const int cl = tid & 63, sg = tid >> 6, c = blockIdx.x * 64 + cl;
    const float *ml = a.part_ml + 2 * qh * a.max_splits;
    const float *po = a.part_o + qh * a.max_splits * D + c;
    constexpr int U = 16;
    float M = -INFINITY, o = 0.0f, L = 0.0f;
    for (int s0 = sg; s0 < nsp; s0 += 4 * U) {
        float mv[U], lv[U], ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s2 = s0 + 4 * u;
            const bool ok = s2 < nsp;
            mv[u] = ok ? ml[2 * s2] : -INFINITY;
            lv[u] = ok ? ml[2 * s2 + 1] : 0.0f;
            ov[u] = ok ? po[(int64_t)s2 * D] : 0.0f;
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < U; ++u) mb = fmaxf(mb, mv[u]);  // finite: split s0 exists
        const float sc = fast_exp2(M - mb);                  // 0 on the first chunk
        o *= sc;
        L *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float e = fast_exp2(mv[u] - mb);
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
        float on = 0.0f, Ln = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float e = fast_exp2(s_m[g][cl] - Mt);  // 0 for a group without splits
            on = fmaf(e, s_o[g][cl], on);
            Ln = fmaf(e, s_l[g][cl], Ln);
        }
        a.out[qh * D + c] = on / Ln;
    }
}

template <int D, int KC, int VC>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
    using C = Cfg<D, KC, VC>;
    const size_t scale_lds = (size_t)C::QOFF + (size_t)a.gqa * D * sizeof(float);
    const size_t merge_lds = (size_t)kWaves * a.gqa * (D + 4 + 2) * sizeof(float);
    const size_t lds = scale_lds > merge_lds ? scale_lds : merge_lds;
    const dim3 grid((unsigned)a.max_splits, (unsigned)a.k.n_kv_heads, (unsigned)a.n_seqs);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_kernel<D, KC, VC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    decode_kernel<D, KC, VC><<<grid, dim3(kThreads), lds, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_splits <= 1) return e;
    combine_kernel<D><<<dim3(D / 64, (unsigned)a.n_q_heads, (unsigned)a.n_seqs), dim3(256), 0, s>>>(a);
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
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

DecodePlan plan_decode(int head_dim, int n_kv_heads, int n_q_heads, int n_seqs, int64_t max_len) {
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
    p.part_ml_bytes = (size_t)n_seqs * n_q_heads * p.max_splits * 2 * sizeof(float);
    p.part_o_bytes = (size_t)n_seqs * n_q_heads * p.max_splits * head_dim * sizeof(float);
    p.off_part_ml = 0;
    p.off_part_o = p.off_part_ml + up(p.part_ml_bytes);
    p.total_bytes = p.off_part_o + up(p.part_o_bytes);
    return p;
}

bool decode_supported(int k_codec, int v_codec, int head_dim) {
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
