/*
 * kvq.h -- C ABI of libkvq: attention over a block-quantized KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are web pages, cited by title/section):
 *   - den_llama.cpp, "What this fork is": the Q4_G64 KV codec (signed INT4 plus
 *     one FP16 scale per 64 values, 4.25 bits/value) with a quantizer that is
 *     byte-identical, and a dequantizer bit-identical, to a CPU reference;
 *     layer-wise split KV precision (some layers keep a wider codec).
 *   - den_llama.cpp, "Results": FlashAttention reading a q8_0 K / q4_0 V cache
 *     directly instead of falling back to f16 ("FA silently falls back" is
 *     presented as the defect to avoid: this library never falls back).
 *   - den_llama.cpp, "What's in the fork": quantize-on-write of new K/V rows
 *     (set-rows / cpy), dequant (convert), FlashAttention over quantized K/V.
 *   - Llaminar, "Graphs and Compute Stages": KV-cache append is a stage that
 *     precedes attention; "GPU Graph Capture": KV counters stay device-owned
 *     during captured execution; "Activation precision": FP32 activations.
 *
 * Codecs (groups of G consecutive channels of one row, one binary16 scale d16
 * per group, dq = (float)d16; codes q_i = clamp(rint(x_i / dq), -Qmax-1, Qmax)
 * with d = amax/Qmax rounded to binary16 nearest-even, saturated at 65504):
 *   KVQ_Q8_0   : G = 32, Qmax = 127, 8-bit two's complement codes  (8.5 b/value)
 *   KVQ_Q4_0   : G = 32, Qmax = 7,   4-bit codes stored as q + 8   (4.5 b/value)
 *   KVQ_Q4_G64 : G = 64, Qmax = 7,   4-bit two's complement codes  (4.25 b/value)
 * Dequantized value: x_hat_i = q_i * dq (exact in binary32).
 *
 * Memory model.  Every pointer argument is a device pointer unless stated;
 * the caller owns all memory (the library never allocates, frees or
 * synchronizes).  Every call only enqueues work on the given HIP stream
 * (NULL = the legacy default stream) and is therefore capturable in a HIP
 * graph.  Argument errors are detected on the host before anything is
 * enqueued; then the call returns a non-zero kvq_status, enqueues nothing and
 * records a message retrievable with kvq_last_error() (thread-local).
 * An unsupported (codec, head_dim, group) combination returns
 * KVQ_EUNSUPPORTED: there is no fallback path.  A failed kernel launch returns
 * KVQ_EHIP.
 *
 * Operand range of the attention calls.  Their matrix-core operands are
 * binary16: decode rounds each dequantized V value x_hat = code * dq to
 * binary16, prefill each K and V value, so |x_hat| must stay within 65504.
 * The block codecs keep every finite input within that unless a group's
 * largest magnitude reaches about 57000 (4-bit codecs) or 65000 (q8_0).  A
 * value beyond it becomes an infinity in the operand and makes every result
 * it can affect non-finite.  Every attention call takes an optional device
 * status word (dev_status, int32, may be NULL): a kernel that writes a
 * non-finite result stores KVQ_EOVERFLOW there (queries must be finite, so a
 * non-finite result can only come from such a value); nothing is stored
 * otherwise, so the caller initializes it.  The status is written by the
 * device, after the call returns.
 *
 * Cache layout (one "plane" = the K or the V cache of one layer).  Rows are
 * grouped in blocks of KVQ_BLOCK_ROWS = 32 consecutive positions of one
 * (sequence, kv-head):
 *   codes  : [n_seqs][n_kv_heads][capacity/32][32 * row_code_bytes]  bytes
 *   scales : [n_seqs][n_kv_heads][capacity/32][32 * head_dim/G]      binary16
 * Inside a block the codes and scales are permuted into the order in which
 * the matrix-core kernels consume them; the permutation depends on the plane's
 * role (KVQ_ROLE_K or KVQ_ROLE_V) and is a pure reordering: the code of row r,
 * channel c is stored exactly once, with the value and bit width the codec
 * defines.  kvq_dequant() returns rows in plain [head][row][channel] order.
 * Both base pointers must be 256-byte aligned.  Rows that were never appended
 * hold whatever the memory held (zero-fill the planes if that matters).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_BLOCK_ROWS 32
#define KVQ_MAX_GQA 16 /* q-heads per kv-head supported by the attention kernels */
#define KVQ_MAX_QUERIES 64 /* queries per sequence in one kvq_attend_decode_mq call */

/* KVQ_F16 is the control the block codecs are measured against (den_llama.cpp,
 * "What this fork is" / "Results": without the quantized FlashAttention pair
 * the fork falls back to an f16 K / f16 V cache): each value stored as its
 * binary16 nearest-even rounding, saturated at +-65504, 16 bits per value,
 * no scales (the scales pointer of an F16 plane may be NULL).  It pairs only
 * with itself (K and V both KVQ_F16), and decode reads it at head_dim 64 and
 * 128; prefill does not read it.  Anything else returns KVQ_EUNSUPPORTED. */
typedef enum { KVQ_Q8_0 = 0, KVQ_Q4_0 = 1, KVQ_Q4_G64 = 2, KVQ_F16 = 3 } kvq_codec;

typedef enum { KVQ_ROLE_K = 0, KVQ_ROLE_V = 1 } kvq_role;

typedef enum {
    KVQ_OK = 0,
    KVQ_EINVAL = 1,       /* bad argument (null pointer, bad size, misalignment, ...) */
    KVQ_EUNSUPPORTED = 2, /* valid but unsupported combination (no fallback exists)   */
    KVQ_ERANGE = 3,       /* a position/length outside the plane's capacity           */
    KVQ_EWORKSPACE = 4,   /* workspace missing or smaller than required               */
    KVQ_EHIP = 5,         /* the HIP runtime reported an error                        */
    KVQ_EOVERFLOW = 6,    /* (device status word) a dequantized K or V value the call  */
                          /* read lies beyond the binary16 range of its operands       */
    KVQ_EWAIT = 7         /* (device status word) a fused append + decode wave's       */
                          /* bounded wait for the appending wave ran out: it went on   */
                          /* and may have read the new rows' old bytes                 */
} kvq_status;

/* One K or V cache plane of one layer.  head_dim must be 64, 128 or 256 and a
 * multiple of the codec's group size; capacity a positive multiple of 32. */
typedef struct {
    int32_t codec;      /* kvq_codec                                         */
    int32_t role;       /* kvq_role: selects the in-block permutation        */
    int32_t head_dim;
    int32_t n_kv_heads;
    int32_t n_seqs;
    int32_t reserved;   /* must be 0                                         */
    int64_t capacity;   /* rows per (sequence, kv-head)                      */
    void *codes;        /* device, 256-B aligned, kvq_plane_bytes() bytes    */
    void *scales;       /* device, 256-B aligned, binary16 bit patterns      */
} kvq_plane;

/* The K and V planes of one layer.  Codecs may differ between k and v (and
 * between layers); head_dim, n_kv_heads, n_seqs and capacity must match;
 * k.role must be KVQ_ROLE_K and v.role KVQ_ROLE_V. */
typedef struct {
    kvq_plane k;
    kvq_plane v;
} kvq_layer;

/* ---- sizing (host only, never touches the GPU) ------------------------- */

/* Code bytes per row: 2*head_dim (KVQ_F16), head_dim (8-bit codec) or
 * head_dim/2 (4-bit codecs); 0 for an invalid codec/head_dim. */
size_t kvq_row_code_bytes(int32_t codec, int32_t head_dim);

/* Bytes of the codes and scales buffers of a plane of the given shape
 * (codes = rows * row_code_bytes, scales = rows * head_dim/G * 2 with
 * rows = n_seqs * n_kv_heads * capacity).  For Q4_G64 the two add up to
 * exactly 4.25 bits per cached value. */
kvq_status kvq_plane_bytes(int32_t codec, int32_t head_dim, int32_t n_kv_heads, int32_t n_seqs,
                           int64_t capacity, size_t *codes_bytes, size_t *scales_bytes);

/* ---- append: quantize new rows into the cache (den_llama.cpp, "What's in the
 * fork": quantize-on-write; Llaminar, "Graphs and Compute Stages": append
 * precedes attention) ----------------------------------------------------- */

/* Quantizes n_tokens new rows per kv-head into L->k and L->v.
 *   k_new, v_new : fp32 [n_tokens][n_kv_heads][head_dim], device; either may
 *                  be NULL to leave that plane untouched (not both).
 *   seq_idx      : int32 [n_tokens], device: the sequence of each token.
 *   pos          : int64 [n_tokens], device: the row (position) of each token.
 *   dev_status   : optional int32, device: if any token has seq_idx outside
 *                  [0, n_seqs) or pos outside [0, capacity) that token is
 *                  skipped and KVQ_ERANGE is stored here (nothing is stored
 *                  otherwise; the caller initializes it).
 * Tokens of one call must target distinct (sequence, position) pairs.
 * Inputs must be finite.  Codes and scales equal the CPU reference bit for
 * bit (den_llama.cpp, "Results": quantizer byte-identical to the CPU ref). */
kvq_status kvq_append(const kvq_layer *L, const float *k_new, const float *v_new,
                      const int32_t *seq_idx, const int64_t *pos, int32_t n_tokens,
                      int32_t *dev_status, void *hip_stream);

/* ---- decode attention (den_llama.cpp, "Results" / "What's in the fork":
 * FlashAttention reading the quantized K/V blocks directly) -------------- */

/* Workspace bytes kvq_attend_decode needs for these sizes (host only). */
size_t kvq_decode_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_seqs,
                                  int64_t max_len);

/* One query per sequence attends rows [0, len_b) of its own cache, with
 * len_b = min(seq_len[b], max_len):
 *   out[b][h] = sum_j softmax_j(softmax_scale * q[b][h] . k_hat[b][g][j]) v_hat[b][g][j]
 * with g = h / (n_q_heads / n_kv_heads) (consecutive q-heads share a kv-head).
 *   q        : fp32 [n_seqs][n_q_heads][head_dim], device
 *   seq_len  : int64 [n_seqs], device (lengths stay device-owned)
 *   max_len  : host upper bound of the lengths, sizes the grid; <= capacity
 *   out      : fp32 [n_seqs][n_q_heads][head_dim], device; zeros for len_b = 0
 *   workspace: device scratch of at least kvq_decode_workspace_bytes() bytes,
 *              256-B aligned; its contents are not preserved across calls and
 *              calls that run concurrently must not share it.
 * n_seqs may be smaller than the planes' n_seqs (sequences 0..n_seqs-1).
 * n_q_heads / n_kv_heads must be an integer in [1, KVQ_MAX_GQA].
 * Precision: fp32 statistics and accumulation; the matrix-core operands are
 * binary16 (query as a hi+lo pair, probabilities and dequantized V rounded to
 * nearest-even); |v_hat| beyond 65504 is reported through dev_status (see
 * "Operand range" above). */
kvq_status kvq_attend_decode(const kvq_layer *L, const float *q, const int64_t *seq_len,
                             int32_t n_seqs, int32_t n_q_heads, int64_t max_len,
                             float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                             int32_t *dev_status, void *hip_stream);

/* ---- multi-query decode (den_llama.cpp, "Ship command": the server drafts
 * up to two tokens per step with multi-token prediction, so a verifying decode
 * step attends from the newest q_len positions at once) ----------------------- */

/* Workspace bytes kvq_attend_decode_mq needs for these sizes (host only). */
size_t kvq_decode_mq_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_seqs,
                                     int32_t q_len, int64_t max_len);

/* q_len queries per sequence, at the newest positions of the sequence: with
 * len_b = min(seq_len[b], max_len), query i (0 <= i < q_len) sits at row
 * p = len_b - q_len + i, whose K/V are already appended, and attends rows
 * [0, p] (causal among the new tokens, itself included):
 *   out[b][i][h] = sum_{j <= p} softmax_j(softmax_scale * q[b][i][h] . k_hat[b][g][j]) v_hat[b][g][j]
 * A query with p < 0 attends nothing: its output is 0.
 *   q   : fp32 [n_seqs][q_len][n_q_heads][head_dim], device
 *   out : fp32 [n_seqs][q_len][n_q_heads][head_dim], device
 *   q_len in [1, KVQ_MAX_QUERIES]; every other argument as for
 *   kvq_attend_decode (which is this call with q_len = 1).
 * Every K/V byte is read once per kv-head for up to 16 / (n_q_heads /
 * n_kv_heads) queries at a time (one launch per such group of queries). */
kvq_status kvq_attend_decode_mq(const kvq_layer *L, const float *q, const int64_t *seq_len,
                                int32_t n_seqs, int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                int32_t *dev_status, void *hip_stream);

/* ---- fused append + decode (den_llama.cpp, "What's in the fork": the
 * quantize-on-write path and the FlashAttention reader of the same codec,
 * which the fork runs as two steps; here one launch does both) ------------ */

/* Appends the step's new token and attends from it, in one launch:
 * with len_b = min(seq_len[b], max_len), row len_b - 1 of every kv-head g of
 * sequence b receives k_new[b][g] / v_new[b][g], quantized exactly as
 * kvq_append stores it, and out is then what kvq_attend_decode returns on
 * the updated cache.  A sequence with len_b <= 0 gets no row and out[b] = 0.
 *   k_new, v_new : fp32 [n_seqs][n_kv_heads][head_dim], device, 16-B aligned
 * Every other argument, the workspace size included, as for
 * kvq_attend_decode.  The appended rows are the only cache bytes written. */
kvq_status kvq_append_attend_decode(const kvq_layer *L, const float *k_new, const float *v_new,
                                    const float *q, const int64_t *seq_len, int32_t n_seqs,
                                    int32_t n_q_heads, int64_t max_len, float softmax_scale, float *out,
                                    void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * kvq_append_attend_decode without the workspace arguments.  The split
 * partials go to a scratch array inside the library's code object, one per
 * GPU, of kvq_noalloc_scratch_bytes() bytes (16 MiB; held until the process
 * ends).  A call whose partials would not fit -- the size
 * kvq_decode_workspace_bytes reports for the same arguments exceeds it --
 * returns KVQ_EWORKSPACE before anything is enqueued.  The call allocates
 * nothing; the first call on a GPU looks the array's address up once.  Every
 * call on one GPU shares that array, so calls that may overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * Every other argument and the result as for kvq_append_attend_decode. */
kvq_status kvq_append_attend_decode_noalloc(const kvq_layer *L, const float *k_new, const float *v_new,
                                            const float *q, const int64_t *seq_len, int32_t n_seqs,
                                            int32_t n_q_heads, int64_t max_len, float softmax_scale, float *out,
                                            int32_t *dev_status, void *hip_stream);
/* The scratch size of kvq_append_attend_decode_noalloc (host only). */
size_t kvq_noalloc_scratch_bytes(void);

/* The same for q_len new tokens per sequence (a verifying multi-query step):
 * rows len_b - q_len + i (those >= 0) receive k_new[b][i] / v_new[b][i], then
 * the call returns what kvq_attend_decode_mq returns on the updated cache.
 *   k_new, v_new : fp32 [n_seqs][q_len][n_kv_heads][head_dim], device
 * Workspace size: kvq_decode_mq_workspace_bytes. */
kvq_status kvq_append_attend_decode_mq(const kvq_layer *L, const float *k_new, const float *v_new,
                                       const float *q, const int64_t *seq_len, int32_t n_seqs,
                                       int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                       float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                       int32_t *dev_status, void *hip_stream);

/* ---- paged planes (den_llama.cpp, "Adaptive KV streaming (contributed)": a
 * bounded device pool of resident KV pages; here the pool itself, addressed
 * through a per-sequence block table, without the host tier) ------------- */

/* A page pool plus the table that maps each sequence's rows to pages.
 *   pool        : k and v planes laid out exactly as contiguous planes whose
 *                 n_seqs is the number of pages and whose capacity is the
 *                 rows per page (a multiple of 32); each page holds those
 *                 rows for every kv-head.
 *   block_table : device int32 [n_seqs][max_pages]; entry [b][i] is the page
 *                 that holds rows [i * page_rows, (i + 1) * page_rows) of
 *                 sequence b.  A sequence's capacity is max_pages * page_rows.
 * Pages need not be distinct across sequences only if the rows they hold are
 * never written through both.  An entry outside [0, pages) makes the
 * attention read zeros for those rows and the append skip them (no memory
 * outside the pool is touched; kvq_paged_append reports KVQ_ERANGE through
 * dev_status). */
typedef struct {
    kvq_layer pool;
    const int32_t *block_table;
    int32_t n_seqs;
    int32_t max_pages;
} kvq_paged_layer;

/* kvq_append through the table: seq_idx in [0, n_seqs), pos in
 * [0, max_pages * page_rows). */
kvq_status kvq_paged_append(const kvq_paged_layer *P, const float *k_new, const float *v_new,
                            const int32_t *seq_idx, const int64_t *pos, int32_t n_tokens, int32_t *dev_status,
                            void *hip_stream);

/* Workspace bytes of the two calls below (host only). */
size_t kvq_paged_decode_workspace_bytes(const kvq_paged_layer *P, int32_t n_q_heads, int32_t n_seqs,
                                        int32_t q_len, int64_t max_len);

/* kvq_attend_decode_mq (q_len = 1: kvq_attend_decode) over paged planes:
 * the same result as on contiguous planes holding the same rows; max_len
 * <= max_pages * page_rows. */
kvq_status kvq_paged_attend_decode_mq(const kvq_paged_layer *P, const float *q, const int64_t *seq_len,
                                      int32_t n_seqs, int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                      float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                      int32_t *dev_status, void *hip_stream);

/* kvq_append_attend_decode_mq over paged planes (the new rows go through
 * the table too). */
kvq_status kvq_paged_append_attend_decode_mq(const kvq_paged_layer *P, const float *k_new, const float *v_new,
                                             const float *q, const int64_t *seq_len, int32_t n_seqs,
                                             int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                             float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                             int32_t *dev_status, void *hip_stream);

/* ---- chunked-prefill attention (den_llama.cpp, "Results": prefill with the
 * quantized cache and 2048-token micro-batches; Llaminar, "GPU Graph
 * Capture": prefill runs in chunks) --------------------------------------- */

/* Workspace bytes kvq_attend_prefill needs (host only). */
size_t kvq_prefill_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_tokens);

/* A chunk of n_tokens queries of sequence `seq` at absolute positions
 * pos0 .. pos0+n_tokens-1, whose K/V rows were already appended; token t
 * attends rows [0, pos0 + t] (causal, itself included).
 *   q_bf16 : bfloat16 bit patterns [n_tokens][n_q_heads][head_dim], device
 *   out    : fp32 [n_tokens][n_q_heads][head_dim], device
 * The dequantized K and V tiles (code * scale) and the probabilities are
 * rounded once to binary16 for the matrix cores; each (token, head) query
 * column is scaled by a power of two (largest value in [1, 2)) before its
 * binary16 rounding, so any bfloat16 magnitude is accepted; accumulation and
 * softmax are fp32.  K and V values beyond the binary16 range are reported
 * through dev_status (see "Operand range" above). */
kvq_status kvq_attend_prefill(const kvq_layer *L, const uint16_t *q_bf16, int32_t seq, int64_t pos0,
                              int32_t n_tokens, int32_t n_q_heads, float softmax_scale, float *out,
                              void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream);

/* kvq_attend_prefill over paged planes (den_llama.cpp, "Adaptive KV streaming
 * (contributed)": the device pool of resident KV pages, read through the
 * sequence's block table): the same result as on contiguous planes holding
 * the same rows.  seq in [0, P->n_seqs); pos0 + n_tokens <= max_pages *
 * page_rows; the pages that the chunk's rows rounded up to a multiple of 64
 * reach must number at most 4096 (else KVQ_EUNSUPPORTED).  Rows whose table
 * entry lies outside the pool read as zeros (key and value 0). */
kvq_status kvq_paged_attend_prefill(const kvq_paged_layer *P, const uint16_t *q_bf16, int32_t seq, int64_t pos0,
                                    int32_t n_tokens, int32_t n_q_heads, float softmax_scale, float *out,
                                    void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream);

/* ---- dequant (den_llama.cpp, "What's in the fork": convert; "Results":
 * dequant bit-identical to the CPU reference) ----------------------------- */

/* Writes x_hat = q * dq for rows [row0, row0 + n_rows) of sequence `seq`:
 *   out : fp32 [n_kv_heads][n_rows][head_dim], device. */
kvq_status kvq_dequant(const kvq_plane *P, int32_t seq, int64_t row0, int64_t n_rows, float *out,
                       void *hip_stream);

/* ---- diagnostics --------------------------------------------------------- */

/* The fused append + decode calls (kvq_append_attend_decode and its
 * variants) let the waves that read the block holding a new row wait, in
 * LDS, for the wave that stores it, at most `polls` polls (default 2^20,
 * far beyond any real delay); a wait that runs out goes on and stores
 * KVQ_EWAIT in the call's dev_status, so no kernel can hang on it.
 * hold_flag != 0 keeps the storing wave from signalling, so that tests can
 * drive that path; it is for tests only.  Applies to calls made after it
 * (process-wide).  KVQ_EINVAL for polls < 0. */
kvq_status kvq_debug_append_wait(int32_t polls, int32_t hold_flag);

const char *kvq_status_str(int32_t status);
/* Message of the last failing call on this thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
