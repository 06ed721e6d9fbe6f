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
//  * All K/V scales of the split are staged in LDS by the whole workgroup up
//    front; code words are prefetched one block ahead in registers.
//  * The 8 waves merge through LDS; each workgroup writes one partial
//    (unnormalized O, max, sum) per query head, or the final output when the
//    sequence fits in one split; combine_kernel merges the splits
//    (log-sum-exp) with all partial loads in flight at once.
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

template <int D, int KC, int VC>
struct BlockCodes {
    uint32_t k[2][Cfg<D, KC, VC>::K_WORDS];
    uint32_t v[Cfg<D, KC, VC>::V_WORDS];
};

template <int D, int KC, int VC>
__device__ __forceinline__ void load_block(BlockCodes<D, KC, VC> &bc, const uint8_t *kblk,
                                           const uint8_t *vblk, int lane) {
    using C = Cfg<D, KC, VC>;
    load_lane_words<C::K_LB>(kblk, lane, bc.k[0]);
    load_lane_words<C::K_LB>(kblk + C::K_TILE_BYTES, lane, bc.k[1]);
    load_lane_words<C::V_LB>(vblk, lane, bc.v);
}

template <int D, int KC, int VC>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
    using C = Cfg<D, KC, VC>;
    extern __shared__ __align__(16) unsigned char smem[];

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
    const int64_t r1 = (r0 + a.split_rows < len) ? r0 + a.split_rows : len;
    const int nblk = (int)((r1 - r0 + kBlockRows - 1) / kBlockRows);
    const int64_t blk0 = r0 / kBlockRows;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane & 15, q4 = lane >> 4;
    const int G = a.gqa;

    const int64_t head_lin = (int64_t)b * a.k.n_kv_heads + kvh;
    const uint8_t *kcodes = a.k.codes + head_lin * a.k.head_code_stride + blk0 * C::K_BLOCK_BYTES;
    const uint8_t *vcodes = a.v.codes + head_lin * a.v.head_code_stride + blk0 * C::V_BLOCK_BYTES;
    const uint16_t *kscales = a.k.scales + head_lin * a.k.head_scale_stride + blk0 * C::K_BLOCK_SCALES;
    const uint16_t *vscales = a.v.scales + head_lin * a.v.head_scale_stride + blk0 * C::V_BLOCK_SCALES;

    // Prefetch this wave's first block of codes.
    BlockCodes<D, KC, VC> cur;
    if (wave < nblk) load_block<D, KC, VC>(cur, kcodes + (int64_t)wave * C::K_BLOCK_BYTES,
                                           vcodes + (int64_t)wave * C::V_BLOCK_BYTES, lane);

    // Stage every K and V scale of the split in LDS (contiguous in memory).
    uint16_t *sk = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sv = sk + (a.split_rows / kBlockRows) * C::K_BLOCK_SCALES;
    {
        const int kw = nblk * C::K_BLOCK_SCALES / 8;  // 16-byte units (block scales are 64k B)
        const int vw = nblk * C::V_BLOCK_SCALES / 8;
        const u4 *ks4 = reinterpret_cast<const u4 *>(kscales);
        const u4 *vs4 = reinterpret_cast<const u4 *>(vscales);
        for (int i = tid; i < kw; i += kThreads) reinterpret_cast<u4 *>(sk)[i] = ks4[i];
        for (int i = tid; i < vw; i += kThreads) reinterpret_cast<u4 *>(sv)[i] = vs4[i];
    }

    // Query operand: this lane's head h, channels 32t + 8*q4 + s of k-step t.
    float qv[C::KSTEPS][8];
    {
        const bool real = h < G;
        const float *qp = a.q + ((int64_t)b * a.n_q_heads + (int64_t)kvh * G + (real ? h : 0)) * D;
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
            const float4 x0 = *reinterpret_cast<const float4 *>(qp + 32 * t + 8 * q4);
            const float4 x1 = *reinterpret_cast<const float4 *>(qp + 32 * t + 8 * q4 + 4);
            qv[t][0] = x0.x; qv[t][1] = x0.y; qv[t][2] = x0.z; qv[t][3] = x0.w;
            qv[t][4] = x1.x; qv[t][5] = x1.y; qv[t][6] = x1.z; qv[t][7] = x1.w;
            if (!real)
#pragma unroll
                for (int s = 0; s < 8; ++s) qv[t][s] = 0.0f;
        }
    }
    float qmaxabs = 0.0f;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t)
#pragma unroll
        for (int s = 0; s < 8; ++s) qmaxabs = fmaxf(qmaxabs, fabsf(qv[t][s]));
    qmaxabs = fmaxf(qmaxabs, shfl_xor(qmaxabs, 16));
    qmaxabs = fmaxf(qmaxabs, shfl_xor(qmaxabs, 32));
    // Power-of-two normalisation keeps the binary16 query halves in range.
    const int qexp = qmaxabs > 0.0f ? ilogbf(qmaxabs) : 0;
    const float qnorm = ldexpf(1.0f, -qexp);
    h8 qhi[C::KSTEPS], qlo[C::KSTEPS];
    double corr_d[C::KNG];
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) corr_d[g] = 0.0;
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float x = qv[t][s] * qnorm * k_slot_factor<KC>(s);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            qhi[t][s] = hi;
            qlo[t][s] = lo;
            corr_d[t / C::STEPS_PER_KGROUP] +=
                ((double)(float)hi + (double)(float)lo) * (double)k_slot_bias<KC>(s);
        }
    }
    float corr[C::KNG];
#pragma unroll
    for (int g = 0; g < C::KNG; ++g) {
        double c = corr_d[g];
        c += __shfl_xor(c, 16, 64);
        c += __shfl_xor(c, 32, 64);
        corr[g] = (float)c;
    }
    const float c_h = a.scale_log2 * ldexpf(1.0f, qexp);

    __syncthreads();  // scales staged
    if ((r1 & (kBlockRows - 1)) != 0) {
        // Rows past the end of the last block may never have been written:
        // zero their V scales so that 0 * V_hat stays 0 whatever the bytes hold.
        uint16_t *svl = sv + (nblk - 1) * C::V_BLOCK_SCALES;
        const int valid = (int)(r1 & (kBlockRows - 1));
        for (int i = tid; i < C::V_BLOCK_SCALES; i += kThreads) {
            const int kq = i / (8 * C::VNG), sl = i % 8;
            const int j = (sl >> 2) * 16 + 4 * kq + (sl & 3);
            if (j >= valid) svl[i] = 0;
        }
        __syncthreads();
    }

    f4 O[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) O[cb] = f4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int bi = wave; bi < nblk; bi += kWaves) {
        BlockCodes<D, KC, VC> nxt;
        const bool more = bi + kWaves < nblk;
        if (more) load_block<D, KC, VC>(nxt, kcodes + (int64_t)(bi + kWaves) * C::K_BLOCK_BYTES,
                                        vcodes + (int64_t)(bi + kWaves) * C::V_BLOCK_BYTES, lane);

        // ---- scores S^T for the two 16-row tiles
        const uint16_t *skb = sk + bi * C::K_BLOCK_SCALES;
        float S[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const _Float16 *ksc = reinterpret_cast<const _Float16 *>(skb + tau * 16 * C::KNG +
                                                                      q4 * 4 * C::KNG);
            float sacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < C::KNG; ++g) {
                f4 acc = f4{-corr[g], -corr[g], -corr[g], -corr[g]};
#pragma unroll
                for (int st = 0; st < C::STEPS_PER_KGROUP; ++st) {
                    const int t = g * C::STEPS_PER_KGROUP + st;
                    const h8 kop = k_operand<KC>(&cur.k[tau][is8(KC) ? 2 * t : t]);
                    acc = mfma16x16x32(kop, qhi[t], acc);
                    acc = mfma16x16x32(kop, qlo[t], acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[r] = fmaf(acc[r], (float)ksc[g * 4 + r], sacc[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) S[tau][r] = sacc[r] * c_h;
        }
        // mask rows past the end of the split
        const int64_t rowbase = r0 + (int64_t)bi * kBlockRows;
        if (rowbase + kBlockRows > r1) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (rowbase + 16 * tau + 4 * q4 + r >= r1) S[tau][r] = -INFINITY;
        }

        // ---- online softmax (log2 domain)
        float mx = S[0][0];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[tau][r]);
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

        // ---- O^T += V^T P^T, one 16-channel block at a time
        const h2 *svb = reinterpret_cast<const h2 *>(sv + bi * C::V_BLOCK_SCALES + q4 * 8 * C::VNG);
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb) {
            const int gv = cb * 16 / C::VG;
            const h8 vop = v_operand<VC>(&cur.v[is8(VC) ? 2 * cb : cb], svb + gv * 4);
            O[cb] = mfma16x16x32(vop, P, O[cb]);
        }
        if (more) cur = nxt;
    }

    // ---- merge the 8 waves through LDS (reuses the scale area)
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    __syncthreads();
    float *so = reinterpret_cast<float *>(smem);           // [wave][G][D]
    float *sm = so + kWaves * G * D;                        // [wave][G]
    float *sl = sm + kWaves * G;                            // [wave][G]
    if (h < G) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) so[(wave * G + h) * D + 16 * cb + 4 * q4 + r] = O[cb][r];
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
            o = fmaf(e, so[(w * G + hh) * D + c], o);
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
// per workgroup: 4 thread groups take every 4th split with independent loads,
// the per-split weights exp2(m_s - M) are computed once into LDS.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
    extern __shared__ float sw[];  // [nsp] weights, then [4][64] partial sums
    __shared__ float s_red[256];
    const int hq = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    int64_t len = a.seq_len[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int nsp = (int)((len + a.split_rows - 1) / a.split_rows);
    if (nsp <= 1) return;  // the decode kernel wrote the output itself
    const int64_t qh = (int64_t)b * a.n_q_heads + hq;
    const float *ml = a.part_ml + 2 * qh * a.max_splits;
    // M = max_s m_s
    float M = -INFINITY;
    for (int s2 = tid; s2 < nsp; s2 += 256) M = fmaxf(M, ml[2 * s2]);
    s_red[tid] = M;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
        __syncthreads();
    }
    M = s_red[0];
    __syncthreads();
    float L = 0.0f;
    for (int s2 = tid; s2 < nsp; s2 += 256) {
        const float w = fast_exp2(ml[2 * s2] - M);
        sw[s2] = w;
        L = fmaf(w, ml[2 * s2 + 1], L);
    }
    s_red[tid] = L;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) s_red[tid] += s_red[tid + w];
        __syncthreads();
    }
    L = s_red[0];
    __syncthreads();
    const int c = blockIdx.x * 64 + (tid & 63), sg = tid >> 6;
    const float *po = a.part_o + qh * a.max_splits * D + c;
    float o = 0.0f;
#pragma unroll 8
    for (int s2 = sg; s2 < nsp; s2 += 4) o = fmaf(sw[s2], po[(int64_t)s2 * D], o);
    s_red[tid] = o;
    __syncthreads();
    if (sg == 0)
        a.out[qh * D + c] = (s_red[tid] + s_red[tid + 64] + s_red[tid + 128] + s_red[tid + 192]) / L;
}

template <int D, int KC, int VC>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
    using C = Cfg<D, KC, VC>;
    const size_t scale_lds = (size_t)(a.split_rows / kBlockRows) *
                             (C::K_BLOCK_SCALES + C::V_BLOCK_SCALES) * sizeof(uint16_t);
    const size_t merge_lds = (size_t)kWaves * a.gqa * (D + 2) * sizeof(float);
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
    combine_kernel<D><<<dim3(D / 64, (unsigned)a.n_q_heads, (unsigned)a.n_seqs), dim3(256),
                        (size_t)a.max_splits * sizeof(float), s>>>(a);
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
