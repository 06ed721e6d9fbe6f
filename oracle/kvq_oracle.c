/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for attention over a
 * block-quantized KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no header, table, helper or constant generator
 * with the GPU path: everything it needs is written out here from the
 * definitions.
 *
 * Sources (web pages, cited by title and section):
 *   [den]  "den_llama.cpp" -- section "What this fork is" (the Q4_G64 KV codec:
 *          signed INT4 with one FP16 scale per 64 values, 4.25 bits/value, and a
 *          byte/bit-exact CPU quantizer/dequantizer), section "Results" /
 *          "build3 additions" (q8_0 K / q4_0 V FlashAttention pair, unit harness
 *          "quantizer byte-identical vs CPU ref, dequant bit-identical"),
 *          section "What's in the fork" (quantize-on-write, dequant, FA over the
 *          quantized cache).
 *   [lla]  "Llaminar" -- section "Graphs and Compute Stages" (KV-cache append
 *          precedes attention), section "Activation precision" (FP32 activations).
 * The block formats of q8_0 and q4_0 are not printed on the pages; the workload
 * statement defines them: q8_0 = 32 int8 + fp16 scale amax/127; q4_0 = 32
 * 4-bit codes with offset 8 + fp16 scale; Q4_G64 = 64 signed int4 in [-8,7] +
 * fp16 scale amax/7, round-to-nearest-even, clamped.  Every reading taken where
 * the pages are silent is listed in the header comment of each function.
 *
 * Floating point: the quantizer runs in IEEE binary32 exactly as written
 * (compile with -O2 -fno-fast-math -ffp-contract=off; x86-64 SSE arithmetic,
 * FLT_EVAL_METHOD == 0); attention runs in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Codec identifiers used by this file's entry points (its own numbering). */
enum { OR_Q8_0 = 0, OR_Q4_0 = 1, OR_Q4_G64 = 2, OR_F16 = 3 };

/* Status codes returned by the entry points. */
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_NONFINITE = 2 };

/* ------------------------------------------------------------------------- */
/* IEEE binary16 conversions, written from the format definition.            */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;        */
/* subnormals are f * 2^-24 for integer f in [1, 1023].                      */
/* ------------------------------------------------------------------------- */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Shift an unsigned integer right by s bits with round-half-to-even. */
static uint64_t shift_rne(uint64_t v, int s)
{
    if (s <= 0) return v << (-s);
    if (s >= 64) return 0;
    uint64_t q = v >> s;
    uint64_t rem = v & ((((uint64_t)1) << s) - 1);
    uint64_t half = ((uint64_t)1) << (s - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
    return q;
}

/* binary32 -> binary16, round to nearest even, subnormals kept, overflow to
 * infinity, NaN stays NaN. */
uint16_t kvq_oracle_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e32 = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (e32 == 0xFF) /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (frac ? 0x0200u : 0u));
    if (e32 == 0) /* zero or binary32 subnormal: far below 2^-25, rounds to 0 */
        return sign;

    /* x = sig * 2^(e32 - 150) with sig a 24-bit integer. */
    uint64_t sig = (uint64_t)(frac | 0x800000u);
    int e = (int)e32 - 127; /* unbiased exponent of the leading bit */

    if (e >= -14) {
        /* Normal range candidate: keep 11 significant bits. */
        uint64_t m = shift_rne(sig, 13); /* in [2^10, 2^11] */
        int he = e + 15;
        if (m == (1u << 11)) { m >>= 1; he += 1; }
        if (he >= 31) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | ((uint32_t)he << 10) | (uint32_t)(m & 0x3FFu));
    }
    /* Subnormal range: result f * 2^-24, f = x / 2^-24 = sig * 2^(e - 23 + 24). */
    uint64_t f = shift_rne(sig, -(e + 1));
    /* f may reach 1024, which is exactly the encoding of the smallest normal. */
    return (uint16_t)(sign | (uint32_t)f);
}

/* Element-wise binary32 -> binary16 over an array (for exhaustive checks). */
void kvq_oracle_f32_to_f16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = kvq_oracle_f32_to_f16(x[i]);
}

/* binary16 -> binary32 (exact). */
float kvq_oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t f = (uint32_t)h & 0x3FFu;
    float mag;
    if (e == 0x1F)
        return bits_f32(sign | 0x7F800000u | (f << 13));
    if (e == 0)
        mag = (float)f * 0x1p-24f;                 /* exact: f < 2^10 */
    else
        mag = (float)(f | 0x400u) * ldexpf(1.0f, (int)e - 25); /* exact */
    return bits_f32(sign | f32_bits(mag));
}

/* ------------------------------------------------------------------------- */
/* Codec parameters.                                                          */
/* ------------------------------------------------------------------------- */

static int codec_group(int codec)
{
    return codec == OR_Q4_G64 ? 64 : (codec == OR_Q8_0 || codec == OR_Q4_0) ? 32 : 0;
}
static int codec_qmax(int codec) { return codec == OR_Q8_0 ? 127 : 7; }
static int codec_bits(int codec) { return codec == OR_F16 ? 16 : codec == OR_Q8_0 ? 8 : 4; }

/* Bytes of codes per row of d values. */
int64_t kvq_oracle_row_code_bytes(int codec, int d)
{
    return (int64_t)d * codec_bits(codec) / 8;
}

/* ------------------------------------------------------------------------- */
/* The f16 control codec ([den] "What this fork is" / "Results": without the */
/* quantized FlashAttention pair compiled in, the fork's golden build falls   */
/* back to an f16 K / f16 V cache, the control the q8_0 K / q4_0 V build is   */
/* measured against).  Each value is stored as its binary16 nearest-even      */
/* rounding, two bytes little-endian, with no scales.  Reading where the      */
/* pages are silent: values beyond the binary16 range saturate at +-65504     */
/* (the rule the block codecs apply to their scales), so the cache stays      */
/* finite.                                                                   */
/* ------------------------------------------------------------------------- */

static int f16_rows(int d, int64_t n_rows, const float *x, uint8_t *codes)
{
    for (int64_t i = 0; i < n_rows * (int64_t)d; ++i) {
        float v = x[i];
        if (!isfinite(v)) return OR_NONFINITE;
        if (v > 65504.0f) v = 65504.0f;
        if (v < -65504.0f) v = -65504.0f;
        uint16_t h = kvq_oracle_f32_to_f16(v);
        codes[2 * i] = (uint8_t)(h & 0xFFu);
        codes[2 * i + 1] = (uint8_t)(h >> 8);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Quantizer for one group of G values ([den] "What this fork is"; workload   */
/* statement for the scale rule).                                             */
/*                                                                           */
/*  1. amax = max |x_i|                          (exact in binary32)          */
/*  2. d    = amax / Qmax                        (one IEEE binary32 divide)   */
/*  3. d16  = binary16_RNE(min(d, 65504))        (stored scale)               */
/*  4. dq   = (float) d16                                                     */
/*  5. q_i  = 0 if dq == 0, else clamp(rint(x_i / dq), -Qmax-1, Qmax)          */
/*                                                                           */
/* Readings where the pages are silent: the code divides by the rounded      */
/* scale dq (that is the value dequantization multiplies by); the divide is  */
/* the IEEE one, not a reciprocal-multiply; rounding is half-to-even for all  */
/* three codecs; q4_0 uses the same symmetric amax/7 rule as Q4_G64 with the  */
/* stored nibble q+8; inputs must be finite.                                  */
/* ------------------------------------------------------------------------- */
int kvq_oracle_quantize_group(int codec, const float *x, uint16_t *scale_bits, int32_t *q)
{
    int G = codec_group(codec);
    if (G == 0) return OR_BAD_ARG;
    int qmax = codec_qmax(codec);

    float amax = 0.0f;
    for (int i = 0; i < G; ++i) {
        if (!isfinite(x[i])) return OR_NONFINITE;
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float d = amax / (float)qmax;
    if (d > 65504.0f) d = 65504.0f;
    uint16_t d16 = kvq_oracle_f32_to_f16(d);
    float dq = kvq_oracle_f16_to_f32(d16);
    *scale_bits = d16;
    for (int i = 0; i < G; ++i) {
        if (dq == 0.0f) { q[i] = 0; continue; }
        float r = rintf(x[i] / dq);
        if (r < (float)(-qmax - 1)) r = (float)(-qmax - 1);
        if (r > (float)qmax) r = (float)qmax;
        q[i] = (int32_t)r;
    }
    return OR_OK;
}

/* Storage of one row's codes ([den] "What this fork is": signed INT4 for
 * Q4_G64; q8_0 as int8 and q4_0 as 4-bit codes with offset 8, the storage
 * of those two codecs that the page names beside it).
 * Logical row layout used by the oracle:
 *   q8_0   : byte i = two's complement int8 of q_i
 *   q4_0   : nibble i = q_i + 8
 *   Q4_G64 : nibble i = q_i & 0xF (two's complement int4)
 *   4-bit packing: byte j = nibble(2j) | nibble(2j+1) << 4.
 * Scales: one binary16 per group, group g covering values [g*G, (g+1)*G). */
int kvq_oracle_quantize_rows(int codec, int d, int64_t n_rows, const float *x,
                             uint8_t *codes, uint16_t *scales)
{
    if (codec == OR_F16) return d > 0 && n_rows >= 0 ? f16_rows(d, n_rows, x, codes) : OR_BAD_ARG;
    int G = codec_group(codec);
    if (G == 0 || d <= 0 || d % G != 0 || n_rows < 0) return OR_BAD_ARG;
    int ng = d / G;
    int64_t rb = kvq_oracle_row_code_bytes(codec, d);
    int32_t q[64];
    for (int64_t r = 0; r < n_rows; ++r) {
        const float *xr = x + r * (int64_t)d;
        uint8_t *cr = codes + r * rb;
        for (int g = 0; g < ng; ++g) {
            int st = kvq_oracle_quantize_group(codec, xr + g * G, &scales[r * ng + g], q);
            if (st != OR_OK) return st;
            for (int i = 0; i < G; ++i) {
                int c = g * G + i;
                if (codec == OR_Q8_0) {
                    cr[c] = (uint8_t)(int8_t)q[i];
                } else {
                    uint8_t nib = codec == OR_Q4_0 ? (uint8_t)(q[i] + 8) : (uint8_t)(q[i] & 0xF);
                    if (c % 2 == 0) cr[c / 2] = (uint8_t)((cr[c / 2] & 0xF0u) | nib);
                    else            cr[c / 2] = (uint8_t)((cr[c / 2] & 0x0Fu) | (nib << 4));
                }
            }
        }
    }
    return OR_OK;
}

/* Dequantization: x_hat_i = (float) q_i * dq.  The product of an integer of at
 * most 8 bits and an 11-bit significand fits in 24 bits, so it is exact in
 * binary32 ([den] "Results": dequant bit-identical to the CPU reference). */
int kvq_oracle_dequant_rows(int codec, int d, int64_t n_rows, const uint8_t *codes,
                            const uint16_t *scales, float *out)
{
    if (codec == OR_F16) {
        if (d <= 0 || n_rows < 0) return OR_BAD_ARG;
        for (int64_t i = 0; i < n_rows * (int64_t)d; ++i)
            out[i] = kvq_oracle_f16_to_f32((uint16_t)(codes[2 * i] | (codes[2 * i + 1] << 8)));
        return OR_OK;
    }
    int G = codec_group(codec);
    if (G == 0 || d <= 0 || d % G != 0 || n_rows < 0) return OR_BAD_ARG;
    int ng = d / G;
    int64_t rb = kvq_oracle_row_code_bytes(codec, d);
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint8_t *cr = codes + r * rb;
        for (int c = 0; c < d; ++c) {
            int qi;
            if (codec == OR_Q8_0) {
                qi = (int8_t)cr[c];
            } else {
                int nib = (c % 2 == 0) ? (cr[c / 2] & 0xF) : (cr[c / 2] >> 4);
                qi = codec == OR_Q4_0 ? nib - 8 : (nib >= 8 ? nib - 16 : nib);
            }
            float dq = kvq_oracle_f16_to_f32(scales[r * ng + c / G]);
            out[r * (int64_t)d + c] = (float)qi * dq;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Attention (binary64).                                                      */
/* ------------------------------------------------------------------------- */

/* Softmax attention of one query vector over rows [0, n) of one KV head:
 *   s_j = scale * sum_c q_c k_jc;  m = max_j s_j;
 *   o   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m)
 * An empty row range gives the zero vector (reading: FlashAttention's usual
 * convention; the pages do not cover it). */
static void attend_one(int d, const float *qv, const float *k, const float *v,
                       int64_t n, double scale, double *s_buf, float *out)
{
    if (n <= 0) {
        for (int c = 0; c < d; ++c) out[c] = 0.0f;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        const float *kj = k + j * (int64_t)d;
        for (int c = 0; c < d; ++c) acc += (double)qv[c] * (double)kj[c];
        s_buf[j] = scale * acc;
        if (s_buf[j] > m) m = s_buf[j];
    }
    double denom = 0.0;
    double *o = (double *)calloc((size_t)d, sizeof(double));
    for (int64_t j = 0; j < n; ++j) {
        double p = exp(s_buf[j] - m);
        denom += p;
        const float *vj = v + j * (int64_t)d;
        for (int c = 0; c < d; ++c) o[c] += p * (double)vj[c];
    }
    for (int c = 0; c < d; ++c) out[c] = (float)(o[c] / denom);
    free(o);
}

/* Decode attention for one sequence ([den] "What's in the fork": the
 * FlashAttention path reads the quantized K/V cache; here K and V are the
 * dequantized rows, which are exact).
 *   q     : [n_q_heads][d]                 fp32 queries
 *   k, v  : [n_kv_heads][row_stride][d]    dequantized rows, rows [0, len) used
 *   out   : [n_sel][d]                     one output per selected q-head
 * GQA reading: q-head h reads kv-head h / (n_q_heads / n_kv_heads). */
int kvq_oracle_attend_decode(int d, int n_q_heads, int n_kv_heads, int64_t len,
                             int64_t row_stride, const float *q, const float *k,
                             const float *v, double scale, const int32_t *sel_heads,
                             int n_sel, float *out)
{
    if (d <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || len < 0 || len > row_stride)
        return OR_BAD_ARG;
    int group = n_q_heads / n_kv_heads;
    double *s = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
    for (int i = 0; i < n_sel; ++i) {
        int h = sel_heads[i];
        if (h < 0 || h >= n_q_heads) { free(s); return OR_BAD_ARG; }
        int g = h / group;
        attend_one(d, q + (int64_t)h * d, k + (int64_t)g * row_stride * d,
                   v + (int64_t)g * row_stride * d, len, scale, s, out + (int64_t)i * d);
    }
    free(s);
    return OR_OK;
}

/* Chunked-prefill attention for one sequence: the chunk's T tokens sit at
 * absolute positions P..P+T-1 and were appended to the cache before attending
 * ([lla] "Graphs and Compute Stages": KV-cache append, then attention).
 * Token t attends rows [0, P + t] inclusive (causal, including itself).
 *   q   : [T][n_q_heads][d]  (bf16 queries widened exactly to fp32)
 *   k,v : [n_kv_heads][row_stride][d] dequantized rows
 *   sel_tok, sel_head : n_sel (token, head) pairs to evaluate
 *   out : [n_sel][d] */
int kvq_oracle_attend_prefill(int d, int n_q_heads, int n_kv_heads, int64_t P, int T,
                              int64_t row_stride, const float *q, const float *k,
                              const float *v, double scale, const int32_t *sel_tok,
                              const int32_t *sel_head, int n_sel, float *out)
{
    if (d <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || P < 0 || T < 0 ||
        P + T > row_stride)
        return OR_BAD_ARG;
    int group = n_q_heads / n_kv_heads;
    double *s = (double *)malloc(sizeof(double) * (size_t)(P + T > 0 ? P + T : 1));
    for (int i = 0; i < n_sel; ++i) {
        int t = sel_tok[i], h = sel_head[i];
        if (t < 0 || t >= T || h < 0 || h >= n_q_heads) { free(s); return OR_BAD_ARG; }
        int g = h / group;
        attend_one(d, q + ((int64_t)t * n_q_heads + h) * d, k + (int64_t)g * row_stride * d,
                   v + (int64_t)g * row_stride * d, P + t + 1, scale, s, out + (int64_t)i * d);
    }
    free(s);
    return OR_OK;
}
