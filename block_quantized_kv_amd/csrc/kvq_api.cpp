// kvq_api.cpp -- the C ABI declared in include/kvq.h: argument validation on
// the host, workspace sizing, and dispatch to the gfx950 kernels.  Nothing here
// allocates, frees or synchronizes; on any argument error nothing is enqueued.
#include "kvq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kvq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kvq_status fail(kvq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

kvq_status ok() {
    g_last_error[0] = '\0';
    return KVQ_OK;
}

bool codec_valid(int32_t c) { return c == KVQ_Q8_0 || c == KVQ_Q4_0 || c == KVQ_Q4_G64 || c == KVQ_F16; }
bool head_dim_valid(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

kvq_status check_plane(const kvq_plane *P, const char *name, int32_t role) {
    if (!P) return fail(KVQ_EINVAL, "%s: null plane", name);
    if (!codec_valid(P->codec)) return fail(KVQ_EINVAL, "%s: unknown codec %d", name, P->codec);
    if (P->role != role)
        return fail(KVQ_EINVAL, "%s: role %d, expected %d", name, P->role, role);
    if (!head_dim_valid(P->head_dim))
        return fail(KVQ_EUNSUPPORTED, "%s: head_dim %d not in {64,128,256}", name, P->head_dim);
    if (P->head_dim % kvq::group_size(P->codec) != 0)
        return fail(KVQ_EINVAL, "%s: head_dim %d not a multiple of the group", name, P->head_dim);
    if (P->n_kv_heads <= 0 || P->n_seqs <= 0)
        return fail(KVQ_EINVAL, "%s: n_kv_heads=%d n_seqs=%d", name, P->n_kv_heads, P->n_seqs);
    if (P->capacity <= 0 || P->capacity % KVQ_BLOCK_ROWS != 0)
        return fail(KVQ_EINVAL, "%s: capacity %lld not a positive multiple of %d", name,
                    (long long)P->capacity, KVQ_BLOCK_ROWS);
    if (P->reserved != 0) return fail(KVQ_EINVAL, "%s: reserved field must be 0", name);
    if (!P->codes || (!P->scales && P->codec != KVQ_F16)) return fail(KVQ_EINVAL, "%s: null codes/scales", name);
    if (!aligned(P->codes, 256) || !aligned(P->scales, 256))
        return fail(KVQ_EINVAL, "%s: codes/scales not 256-byte aligned", name);
    return KVQ_OK;
}

kvq_status check_layer(const kvq_layer *L) {
    if (!L) return fail(KVQ_EINVAL, "null layer");
    kvq_status st = check_plane(&L->k, "k", KVQ_ROLE_K);
    if (st != KVQ_OK) return st;
    st = check_plane(&L->v, "v", KVQ_ROLE_V);
    if (st != KVQ_OK) return st;
    if (L->k.head_dim != L->v.head_dim || L->k.n_kv_heads != L->v.n_kv_heads ||
        L->k.n_seqs != L->v.n_seqs || L->k.capacity != L->v.capacity)
        return fail(KVQ_EINVAL, "k and v planes differ in shape");
    return KVQ_OK;
}

// the fused append's wait bound (polls) and its test switch
std::atomic<int> g_append_wait_polls{1 << 20};
std::atomic<int> g_hold_append_flag{0};

kvq::PlaneView view(const kvq_plane &P) {
    kvq::PlaneView v;
    v.codes = static_cast<uint8_t *>(P.codes);
    v.scales = static_cast<uint16_t *>(P.scales);
    v.codec = P.codec;
    v.head_dim = P.head_dim;
    v.n_kv_heads = P.n_kv_heads;
    v.n_seqs = P.n_seqs;
    v.capacity = P.capacity;
    const int64_t blocks = P.capacity / KVQ_BLOCK_ROWS;
    v.head_code_stride = blocks * kvq::block_code_bytes(P.codec, P.head_dim);
    v.head_scale_stride = blocks * kvq::block_scales(P.codec, P.head_dim);
    return v;
}

kvq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(KVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace kvq {
void set_append_wait(int polls, int hold_flag) {
    g_append_wait_polls.store(polls);
    g_hold_append_flag.store(hold_flag);
}
void get_append_wait(int *polls, int *hold_flag) {
    *polls = g_append_wait_polls.load();
    *hold_flag = g_hold_append_flag.load();
}
}  // namespace kvq

extern "C" {

kvq_status kvq_debug_append_wait(int32_t polls, int32_t hold_flag) {
    if (polls < 0) return fail(KVQ_EINVAL, "polls %d < 0", polls);
    kvq::set_append_wait(polls, hold_flag ? 1 : 0);
    return ok();
}

size_t kvq_row_code_bytes(int32_t codec, int32_t head_dim) {
    if (!codec_valid(codec) || head_dim <= 0 || head_dim % kvq::group_size(codec) != 0) return 0;
    return (size_t)kvq::row_bytes(codec, head_dim);
}

kvq_status kvq_plane_bytes(int32_t codec, int32_t head_dim, int32_t n_kv_heads, int32_t n_seqs,
                           int64_t capacity, size_t *codes_bytes, size_t *scales_bytes) {
    if (!codes_bytes || !scales_bytes) return fail(KVQ_EINVAL, "null output pointer");
    if (!codec_valid(codec)) return fail(KVQ_EINVAL, "unknown codec %d", codec);
    if (!head_dim_valid(head_dim))
        return fail(KVQ_EUNSUPPORTED, "head_dim %d not in {64,128,256}", head_dim);
    if (n_kv_heads <= 0 || n_seqs <= 0 || capacity <= 0 || capacity % KVQ_BLOCK_ROWS != 0)
        return fail(KVQ_EINVAL, "bad plane shape");
    const size_t rows = (size_t)n_kv_heads * (size_t)n_seqs * (size_t)capacity;
    *codes_bytes = rows * (size_t)kvq::row_bytes(codec, head_dim);
    *scales_bytes = rows * (size_t)kvq::n_groups(codec, head_dim) * 2;
    return ok();
}

namespace {

// The page table of a paged layer (table null: contiguous planes).
kvq::PageTable no_pages() {
    kvq::PageTable t;
    t.table = nullptr;
    t.table_stride = 0;
    t.page_rows = 0;
    t.n_seqs = 0;
    return t;
}

kvq_status check_paged(const kvq_paged_layer *P, kvq::PageTable *pt) {
    if (!P) return fail(KVQ_EINVAL, "null paged layer");
    kvq_status st = check_layer(&P->pool);
    if (st != KVQ_OK) return st;
    if (!P->block_table || !aligned(P->block_table, 4)) return fail(KVQ_EINVAL, "null or misaligned block_table");
    if (P->n_seqs <= 0 || P->max_pages <= 0)
        return fail(KVQ_EINVAL, "paged layer: n_seqs=%d max_pages=%d", P->n_seqs, P->max_pages);
    if (P->pool.k.capacity > INT32_MAX) return fail(KVQ_EUNSUPPORTED, "page of 2^31 rows or more");
    pt->table = P->block_table;
    pt->table_stride = P->max_pages;
    pt->page_rows = (int)P->pool.k.capacity;
    pt->n_seqs = P->n_seqs;
    return KVQ_OK;
}

kvq_status append_impl(const kvq_layer *L, const kvq::PageTable &pt, const float *k_new, const float *v_new,
                       const int32_t *seq_idx, const int64_t *pos, int32_t n_tokens, int32_t *dev_status,
                       void *hip_stream) {
    if (n_tokens < 0) return fail(KVQ_EINVAL, "n_tokens %d < 0", n_tokens);
    if (!k_new && !v_new) return fail(KVQ_EINVAL, "both k_new and v_new are null");
    if (n_tokens > 0 && (!seq_idx || !pos)) return fail(KVQ_EINVAL, "null seq_idx/pos");
    if ((k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)))
        return fail(KVQ_EINVAL, "k_new/v_new not 16-byte aligned");
    if (!kvq::append_supported(L->k.codec, L->v.codec))
        return fail(KVQ_EUNSUPPORTED, "codec pair %d/%d: f16 pairs only with f16", L->k.codec, L->v.codec);
    if (n_tokens == 0) return ok();
    kvq::AppendArgs a;
    a.plane[0] = view(L->k);
    a.plane[1] = view(L->v);
    a.pt = pt;
    a.x[0] = k_new;
    a.x[1] = v_new;
    a.seq_idx = seq_idx;
    a.pos = pos;
    a.n_tokens = n_tokens;
    a.dev_status = dev_status;
    return hip_status(kvq::launch_append(a, static_cast<hipStream_t>(hip_stream)), "append launch");
}

}  // namespace

kvq_status kvq_append(const kvq_layer *L, const float *k_new, const float *v_new,
                      const int32_t *seq_idx, const int64_t *pos, int32_t n_tokens,
                      int32_t *dev_status, void *hip_stream) {
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return append_impl(L, no_pages(), k_new, v_new, seq_idx, pos, n_tokens, dev_status, hip_stream);
}

kvq_status kvq_paged_append(const kvq_paged_layer *P, const float *k_new, const float *v_new,
                            const int32_t *seq_idx, const int64_t *pos, int32_t n_tokens, int32_t *dev_status,
                            void *hip_stream) {
    kvq::PageTable pt;
    kvq_status st = check_paged(P, &pt);
    if (st != KVQ_OK) return st;
    return append_impl(&P->pool, pt, k_new, v_new, seq_idx, pos, n_tokens, dev_status, hip_stream);
}

namespace {

// Queries per launch: the (query, head) columns of one kv-head fill at most
// the 16 columns of a matrix-core tile.
int queries_per_launch(int gqa, int q_len) {
    const int per = KVQ_MAX_GQA / gqa;
    return q_len < per ? q_len : per;
}

size_t decode_ws_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_seqs, int32_t q_len,
                       int64_t max_len) {
    if (!L || n_q_heads <= 0 || n_seqs <= 0 || q_len <= 0 || max_len < 0 || L->k.n_kv_heads <= 0 ||
        n_q_heads % L->k.n_kv_heads != 0)
        return 0;
    const int gqa = n_q_heads / L->k.n_kv_heads;
    if (gqa > KVQ_MAX_GQA) return 0;
    const kvq::DecodePlan p = kvq::plan_decode(L->k.head_dim, L->k.n_kv_heads, n_q_heads, n_seqs, max_len,
                                               queries_per_launch(gqa, q_len));
    return p.total_bytes;
}

// app_k / app_v (both null, or both set): fused append of q_len new rows per
// sequence before the attention (the first launch writes them).
// pt: the page table of a paged layer (table null: contiguous planes; the
// caller has checked L).
// static_ws: the partials go to the library's own device scratch (the
// no-allocation entry point; workspace/ws_bytes are ignored).
kvq_status attend_decode(const kvq_layer *L, const kvq::PageTable &pt, const float *app_k, const float *app_v,
                         const float *q, const int64_t *seq_len, int32_t n_seqs, int32_t q_len, int32_t n_q_heads,
                         int64_t max_len, float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                         int32_t *dev_status, void *hip_stream, bool static_ws = false) {
    kvq_status st = KVQ_OK;
    const int32_t seq_limit = pt.table ? pt.n_seqs : L->k.n_seqs;
    const int64_t cap = pt.table ? (int64_t)pt.table_stride * pt.page_rows : L->k.capacity;
    if (!q || !seq_len || !out) return fail(KVQ_EINVAL, "null q/seq_len/out");
    if (!aligned(q, 16) || !aligned(out, 16)) return fail(KVQ_EINVAL, "q/out not 16-byte aligned");
    if ((app_k == nullptr) != (app_v == nullptr)) return fail(KVQ_EINVAL, "k_new and v_new: both or neither");
    if (app_k && (!aligned(app_k, 16) || !aligned(app_v, 16)))
        return fail(KVQ_EINVAL, "k_new/v_new not 16-byte aligned");
    if (n_seqs <= 0 || n_seqs > seq_limit)
        return fail(KVQ_EINVAL, "n_seqs %d outside [1, %d]", n_seqs, seq_limit);
    if (q_len <= 0 || q_len > KVQ_MAX_QUERIES)
        return fail(KVQ_EINVAL, "q_len %d outside [1, %d]", q_len, KVQ_MAX_QUERIES);
    if (n_q_heads <= 0 || n_q_heads % L->k.n_kv_heads != 0)
        return fail(KVQ_EINVAL, "n_q_heads %d not a multiple of n_kv_heads %d", n_q_heads,
                    L->k.n_kv_heads);
    const int gqa = n_q_heads / L->k.n_kv_heads;
    if (gqa > KVQ_MAX_GQA)
        return fail(KVQ_EUNSUPPORTED, "%d q-heads per kv-head exceeds %d", gqa, KVQ_MAX_GQA);
    if (max_len < 0 || max_len > cap)
        return fail(KVQ_ERANGE, "max_len %lld outside [0, capacity %lld]", (long long)max_len, (long long)cap);
    if (!(softmax_scale == softmax_scale)) return fail(KVQ_EINVAL, "softmax_scale is NaN");
    if (!kvq::decode_supported(L->k.codec, L->v.codec, L->k.head_dim))
        return fail(KVQ_EUNSUPPORTED, "no decode kernel for this codec pair/head_dim");
    const size_t need = decode_ws_bytes(L, n_q_heads, n_seqs, q_len, max_len);
    if (static_ws) {
        // every size check above ran before the device is touched
        if (need > kvq::kStaticScratchBytes)
            return fail(KVQ_EWORKSPACE, "this call needs %zu bytes of scratch; the no-allocation entry point "
                        "holds %zu (use the workspace variant)", need, kvq::kStaticScratchBytes);
        st = hip_status(kvq::static_scratch(static_cast<hipStream_t>(hip_stream), &workspace),
                        "locating the library's device scratch");
        if (st != KVQ_OK) return st;
        ws_bytes = kvq::kStaticScratchBytes;
    }
    if (!workspace || ws_bytes < need)
        return fail(KVQ_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    if (!aligned(workspace, 256)) return fail(KVQ_EINVAL, "workspace not 256-byte aligned");

    const int per = queries_per_launch(gqa, q_len);
    const kvq::DecodePlan p =
        kvq::plan_decode(L->k.head_dim, L->k.n_kv_heads, n_q_heads, n_seqs, max_len, per);
    if (p.max_splits > 16384)
        return fail(KVQ_EUNSUPPORTED, "max_len %lld needs %d splits (limit 16384)",
                    (long long)max_len, p.max_splits);
    if ((int64_t)p.max_splits * L->k.n_kv_heads * n_seqs > INT32_MAX)
        return fail(KVQ_EUNSUPPORTED, "%d splits x %d kv-heads x %d sequences exceed one launch",
                    p.max_splits, L->k.n_kv_heads, n_seqs);
    kvq::DecodeArgs a;
    a.k = view(L->k);
    a.v = view(L->v);
    a.pt = pt;
    a.seq_len = seq_len;
    char *ws = static_cast<char *>(workspace);
    a.part_ml = reinterpret_cast<float *>(ws + p.off_part_ml);
    a.part_o = reinterpret_cast<float *>(ws + p.off_part_o);
    a.n_seqs = n_seqs;
    a.n_q_heads = n_q_heads;
    a.gqa = gqa;
    a.max_len = max_len;
    a.split_rows = p.split_rows;
    a.max_splits = p.max_splits;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.dev_status = dev_status;
    kvq::get_append_wait(&a.append_wait_polls, &a.hold_append_flag);
    const int64_t qstride = (int64_t)n_q_heads * L->k.head_dim;  // floats per query
    a.q_seq_stride = (int64_t)q_len * qstride;
    // launches of `per` queries each, in order on the stream (they share the
    // workspace)
    for (int first = 0; first < q_len; first += per) {
        // the first launch appends every new row (later launches' queries
        // see them too)
        a.app_k = first == 0 ? app_k : nullptr;
        a.app_v = first == 0 ? app_v : nullptr;
        a.app_rows = first == 0 && app_k ? q_len : 0;
        a.q_len = q_len - first < per ? q_len - first : per;
        a.q_tail = q_len - first - a.q_len;
        a.q = q + first * qstride;
        a.out = out + first * qstride;
        st = hip_status(kvq::launch_decode(a, static_cast<hipStream_t>(hip_stream)), "decode launch");
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

}  // namespace

size_t kvq_decode_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_seqs,
                                  int64_t max_len) {
    return decode_ws_bytes(L, n_q_heads, n_seqs, 1, max_len);
}

kvq_status kvq_attend_decode(const kvq_layer *L, const float *q, const int64_t *seq_len,
                             int32_t n_seqs, int32_t n_q_heads, int64_t max_len,
                             float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                             int32_t *dev_status, void *hip_stream) {
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_decode(L, no_pages(), nullptr, nullptr, q, seq_len, n_seqs, 1, n_q_heads, max_len, softmax_scale,
                         out, workspace, ws_bytes, dev_status, hip_stream);
}

size_t kvq_decode_mq_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_seqs,
                                     int32_t q_len, int64_t max_len) {
    return decode_ws_bytes(L, n_q_heads, n_seqs, q_len, max_len);
}

kvq_status kvq_attend_decode_mq(const kvq_layer *L, const float *q, const int64_t *seq_len,
                                int32_t n_seqs, int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                int32_t *dev_status, void *hip_stream) {
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_decode(L, no_pages(), nullptr, nullptr, q, seq_len, n_seqs, q_len, n_q_heads, max_len,
                         softmax_scale, out, workspace, ws_bytes, dev_status, hip_stream);
}

kvq_status kvq_append_attend_decode(const kvq_layer *L, const float *k_new, const float *v_new, const float *q,
                                    const int64_t *seq_len, int32_t n_seqs, int32_t n_q_heads, int64_t max_len,
                                    float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                    int32_t *dev_status, void *hip_stream) {
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "null k_new/v_new");
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_decode(L, no_pages(), k_new, v_new, q, seq_len, n_seqs, 1, n_q_heads, max_len, softmax_scale,
                         out, workspace, ws_bytes, dev_status, hip_stream);
}

kvq_status kvq_append_attend_decode_noalloc(const kvq_layer *L, const float *k_new, const float *v_new,
                                            const float *q, const int64_t *seq_len, int32_t n_seqs,
                                            int32_t n_q_heads, int64_t max_len, float softmax_scale, float *out,
                                            int32_t *dev_status, void *hip_stream) {
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "null k_new/v_new");
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_decode(L, no_pages(), k_new, v_new, q, seq_len, n_seqs, 1, n_q_heads, max_len, softmax_scale,
                         out, nullptr, 0, dev_status, hip_stream, true);
}

size_t kvq_noalloc_scratch_bytes(void) { return kvq::kStaticScratchBytes; }

kvq_status kvq_append_attend_decode_mq(const kvq_layer *L, const float *k_new, const float *v_new,
                                       const float *q, const int64_t *seq_len, int32_t n_seqs, int32_t q_len,
                                       int32_t n_q_heads, int64_t max_len, float softmax_scale, float *out,
                                       void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream) {
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "null k_new/v_new");
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_decode(L, no_pages(), k_new, v_new, q, seq_len, n_seqs, q_len, n_q_heads, max_len,
                         softmax_scale, out, workspace, ws_bytes, dev_status, hip_stream);
}

size_t kvq_paged_decode_workspace_bytes(const kvq_paged_layer *P, int32_t n_q_heads, int32_t n_seqs,
                                        int32_t q_len, int64_t max_len) {
    return P ? decode_ws_bytes(&P->pool, n_q_heads, n_seqs, q_len, max_len) : 0;
}

kvq_status kvq_paged_attend_decode_mq(const kvq_paged_layer *P, const float *q, const int64_t *seq_len,
                                      int32_t n_seqs, int32_t q_len, int32_t n_q_heads, int64_t max_len,
                                      float softmax_scale, float *out, void *workspace, size_t ws_bytes,
                                      int32_t *dev_status, void *hip_stream) {
    kvq::PageTable pt;
    kvq_status st = check_paged(P, &pt);
    if (st != KVQ_OK) return st;
    return attend_decode(&P->pool, pt, nullptr, nullptr, q, seq_len, n_seqs, q_len, n_q_heads, max_len,
                         softmax_scale, out, workspace, ws_bytes, dev_status, hip_stream);
}

kvq_status kvq_paged_append_attend_decode_mq(const kvq_paged_layer *P, const float *k_new, const float *v_new,
                                             const float *q, const int64_t *seq_len, int32_t n_seqs, int32_t q_len,
                                             int32_t n_q_heads, int64_t max_len, float softmax_scale, float *out,
                                             void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream) {
    if (!k_new || !v_new) return fail(KVQ_EINVAL, "null k_new/v_new");
    kvq::PageTable pt;
    kvq_status st = check_paged(P, &pt);
    if (st != KVQ_OK) return st;
    return attend_decode(&P->pool, pt, k_new, v_new, q, seq_len, n_seqs, q_len, n_q_heads, max_len,
                         softmax_scale, out, workspace, ws_bytes, dev_status, hip_stream);
}

size_t kvq_prefill_workspace_bytes(const kvq_layer *L, int32_t n_q_heads, int32_t n_tokens) {
    (void)L;
    (void)n_q_heads;
    (void)n_tokens;
    return 0;
}

namespace {

// pt: the page table of a paged layer (table null: contiguous planes; the
// caller has checked L).
kvq_status attend_prefill(const kvq_layer *L, const kvq::PageTable &pt, const uint16_t *q_bf16, int32_t seq,
                          int64_t pos0, int32_t n_tokens, int32_t n_q_heads, float softmax_scale, float *out,
                          int32_t *dev_status, void *hip_stream) {
    const int32_t seq_limit = pt.table ? pt.n_seqs : L->k.n_seqs;
    const int64_t cap = pt.table ? (int64_t)pt.table_stride * pt.page_rows : L->k.capacity;
    if (!q_bf16 || !out) return fail(KVQ_EINVAL, "null q/out");
    if (!aligned(q_bf16, 16) || !aligned(out, 16)) return fail(KVQ_EINVAL, "q/out not 16-byte aligned");
    if (seq < 0 || seq >= seq_limit) return fail(KVQ_EINVAL, "seq %d out of range", seq);
    if (n_tokens < 0) return fail(KVQ_EINVAL, "n_tokens %d < 0", n_tokens);
    if (pos0 < 0 || pos0 + n_tokens > cap)
        return fail(KVQ_ERANGE, "chunk [%lld, %lld) outside capacity %lld", (long long)pos0,
                    (long long)(pos0 + n_tokens), (long long)cap);
    if (pt.table) {
        // the pages the chunk's 64-row tiles touch, kept in LDS by the kernel
        int64_t rows = (pos0 + n_tokens + 63) / 64 * 64;
        rows = rows < cap ? rows : cap;
        const int64_t pages = (rows + pt.page_rows - 1) / pt.page_rows;
        if (pages > kvq::kPrefillMaxPages)
            return fail(KVQ_EUNSUPPORTED, "the chunk reaches %lld pages; paged prefill addresses at most %d",
                        (long long)pages, kvq::kPrefillMaxPages);
    }
    if (pos0 + n_tokens > (int64_t)INT32_MAX)
        return fail(KVQ_EUNSUPPORTED, "prefill positions beyond 2^31 rows");
    if (n_q_heads <= 0 || n_q_heads % L->k.n_kv_heads != 0)
        return fail(KVQ_EINVAL, "n_q_heads %d not a multiple of n_kv_heads %d", n_q_heads,
                    L->k.n_kv_heads);
    const int gqa = n_q_heads / L->k.n_kv_heads;
    // (token, head) columns are int on the device, and one workgroup per 128
    // or more of them per kv-head must fit a one-dimensional grid
    const int64_t ncols = (int64_t)n_tokens * gqa;
    if (ncols > (int64_t)1 << 30 || (ncols + 127) / 128 * L->k.n_kv_heads > (int64_t)INT32_MAX)
        return fail(KVQ_EUNSUPPORTED, "%d tokens x %d q-heads per kv-head x %d kv-heads exceed one launch",
                    n_tokens, gqa, L->k.n_kv_heads);
    if (!(softmax_scale == softmax_scale)) return fail(KVQ_EINVAL, "softmax_scale is NaN");
    if (!kvq::prefill_supported(L->k.codec, L->v.codec, L->k.head_dim))
        return fail(KVQ_EUNSUPPORTED, "no prefill kernel for this codec pair/head_dim");
    if (n_tokens == 0) return ok();
    kvq::PrefillArgs a;
    a.k = view(L->k);
    a.v = view(L->v);
    a.pt = pt;
    a.q = q_bf16;
    a.out = out;
    a.seq = seq;
    a.pos0 = pos0;
    a.n_tokens = n_tokens;
    a.n_q_heads = n_q_heads;
    a.gqa = gqa;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.dev_status = dev_status;
    return hip_status(kvq::launch_prefill(a, static_cast<hipStream_t>(hip_stream)),
                      "prefill launch");
}

}  // namespace

kvq_status kvq_attend_prefill(const kvq_layer *L, const uint16_t *q_bf16, int32_t seq, int64_t pos0,
                              int32_t n_tokens, int32_t n_q_heads, float softmax_scale, float *out,
                              void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream) {
    (void)workspace;
    (void)ws_bytes;
    kvq_status st = check_layer(L);
    if (st != KVQ_OK) return st;
    return attend_prefill(L, no_pages(), q_bf16, seq, pos0, n_tokens, n_q_heads, softmax_scale, out, dev_status, hip_stream);
}

kvq_status kvq_paged_attend_prefill(const kvq_paged_layer *P, const uint16_t *q_bf16, int32_t seq, int64_t pos0,
                                    int32_t n_tokens, int32_t n_q_heads, float softmax_scale, float *out,
                                    void *workspace, size_t ws_bytes, int32_t *dev_status, void *hip_stream) {
    (void)workspace;
    (void)ws_bytes;
    kvq::PageTable pt;
    kvq_status st = check_paged(P, &pt);
    if (st != KVQ_OK) return st;
    return attend_prefill(&P->pool, pt, q_bf16, seq, pos0, n_tokens, n_q_heads, softmax_scale, out, dev_status, hip_stream);
}

kvq_status kvq_dequant(const kvq_plane *P, int32_t seq, int64_t row0, int64_t n_rows, float *out,
                       void *hip_stream) {
    if (!P) return fail(KVQ_EINVAL, "null plane");
    kvq_status st = check_plane(P, "plane", P->role == KVQ_ROLE_V ? KVQ_ROLE_V : KVQ_ROLE_K);
    if (st != KVQ_OK) return st;
    if (!out || !aligned(out, 16)) return fail(KVQ_EINVAL, "out null or not 16-byte aligned");
    if (seq < 0 || seq >= P->n_seqs) return fail(KVQ_EINVAL, "seq %d out of range", seq);
    if (row0 < 0 || n_rows < 0 || row0 + n_rows > P->capacity)
        return fail(KVQ_ERANGE, "rows [%lld, %lld) outside capacity %lld", (long long)row0,
                    (long long)(row0 + n_rows), (long long)P->capacity);
    if (n_rows == 0) return ok();
    kvq::DequantArgs a;
    a.plane = view(*P);
    a.role = P->role;
    a.seq = seq;
    a.row0 = row0;
    a.n_rows = n_rows;
    a.out = out;
    return hip_status(kvq::launch_dequant(a, static_cast<hipStream_t>(hip_stream)),
                      "dequant launch");
}

const char *kvq_status_str(int32_t status) {
    switch (status) {
        case KVQ_OK: return "KVQ_OK";
        case KVQ_EINVAL: return "KVQ_EINVAL: invalid argument";
        case KVQ_EUNSUPPORTED: return "KVQ_EUNSUPPORTED: unsupported combination (no fallback)";
        case KVQ_ERANGE: return "KVQ_ERANGE: position or length outside the capacity";
        case KVQ_EWORKSPACE: return "KVQ_EWORKSPACE: workspace missing or too small";
        case KVQ_EHIP: return "KVQ_EHIP: HIP runtime error";
        case KVQ_EOVERFLOW: return "KVQ_EOVERFLOW: a dequantized value beyond the binary16 operand range";
        case KVQ_EWAIT: return "KVQ_EWAIT: the fused append's bounded wait ran out";
        default: return "unknown kvq_status";
    }
}

const char *kvq_last_error(void) { return g_last_error; }

}  // extern "C"
