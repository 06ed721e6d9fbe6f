/* decode_step.c -- the library's C ABI used from plain C, with no Python in
 * between: a cache is built with kvq_append, then one decode step appends the
 * newest row and attends over every row (kvq_append_attend_decode), as a
 * serving loop written in C would.
 *
 * usage: decode_step DIR K_CODEC V_CODEC HEAD_DIM N_KV_HEADS N_Q_HEADS CONTEXT SCALE
 *   DIR/k.f32, DIR/v.f32 : fp32 [CONTEXT][N_KV_HEADS][HEAD_DIM], the rows of
 *                          one sequence (row CONTEXT-1 is the step's new row)
 *   DIR/q.f32            : fp32 [N_Q_HEADS][HEAD_DIM], the step's query
 * writes DIR/out.f32 (fp32 [N_Q_HEADS][HEAD_DIM]) and prints the device
 * status words; exits non-zero on any library or runtime error. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq.h"

#define CHECK_HIP(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));             \
            exit(2);                                                               \
        }                                                                          \
    } while (0)

#define CHECK_KVQ(call)                                                            \
    do {                                                                           \
        kvq_status s_ = (call);                                                    \
        if (s_ != KVQ_OK) {                                                        \
            fprintf(stderr, "%s: %s (%s)\n", #call, kvq_status_str(s_), kvq_last_error()); \
            exit(3);                                                               \
        }                                                                          \
    } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        perror(path);
        exit(4);
    }
    void *p = malloc(bytes);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "%s: short read\n", path);
        exit(4);
    }
    fclose(f);
    return p;
}

static void *to_device(const void *host, size_t bytes) {
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes));
    CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* one plane: codes and scales sized by the library, zero-filled */
static kvq_plane make_plane(int32_t codec, int32_t role, int32_t d, int32_t heads, int64_t cap) {
    kvq_plane p;
    size_t cb = 0, sb = 0;
    memset(&p, 0, sizeof p);
    CHECK_KVQ(kvq_plane_bytes(codec, d, heads, 1, cap, &cb, &sb));
    p.codec = codec;
    p.role = role;
    p.head_dim = d;
    p.n_kv_heads = heads;
    p.n_seqs = 1;
    p.capacity = cap;
    CHECK_HIP(hipMalloc(&p.codes, cb));
    CHECK_HIP(hipMemset(p.codes, 0, cb));
    if (sb) {
        CHECK_HIP(hipMalloc(&p.scales, sb));
        CHECK_HIP(hipMemset(p.scales, 0, sb));
    }
    return p;
}

int main(int argc, char **argv) {
    if (argc != 9) {
        fprintf(stderr, "usage: %s DIR K_CODEC V_CODEC HEAD_DIM N_KV_HEADS N_Q_HEADS CONTEXT SCALE\n", argv[0]);
        return 1;
    }
    const char *dir = argv[1];
    const int32_t kc = atoi(argv[2]), vc = atoi(argv[3]), d = atoi(argv[4]);
    const int32_t hkv = atoi(argv[5]), hq = atoi(argv[6]);
    const int64_t n = atoll(argv[7]);
    const float scale = (float)atof(argv[8]);
    if (n < 1 || hkv < 1 || hq < 1 || d < 1) return 1;
    const int64_t cap = (n + KVQ_BLOCK_ROWS - 1) / KVQ_BLOCK_ROWS * KVQ_BLOCK_ROWS;
    const size_t row_floats = (size_t)hkv * d;

    float *k = read_file(dir, "k.f32", (size_t)n * row_floats * sizeof(float));
    float *v = read_file(dir, "v.f32", (size_t)n * row_floats * sizeof(float));
    float *q = read_file(dir, "q.f32", (size_t)hq * d * sizeof(float));

    kvq_layer L;
    L.k = make_plane(kc, KVQ_ROLE_K, d, hkv, cap);
    L.v = make_plane(vc, KVQ_ROLE_V, d, hkv, cap);

    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    int32_t *status = NULL;
    CHECK_HIP(hipMalloc((void **)&status, 2 * sizeof(int32_t)));
    CHECK_HIP(hipMemset(status, 0, 2 * sizeof(int32_t)));

    /* the prefix: rows 0 .. n-2 of sequence 0 */
    const int32_t np = (int32_t)(n - 1);
    if (np > 0) {
        int32_t *seq = calloc((size_t)np, sizeof(int32_t));
        int64_t *pos = malloc((size_t)np * sizeof(int64_t));
        for (int32_t i = 0; i < np; ++i) pos[i] = i;
        float *dk = to_device(k, (size_t)np * row_floats * sizeof(float));
        float *dv = to_device(v, (size_t)np * row_floats * sizeof(float));
        int32_t *dseq = to_device(seq, (size_t)np * sizeof(int32_t));
        int64_t *dpos = to_device(pos, (size_t)np * sizeof(int64_t));
        CHECK_KVQ(kvq_append(&L, dk, dv, dseq, dpos, np, status, s));
        CHECK_HIP(hipStreamSynchronize(s));
        CHECK_HIP(hipFree(dk));
        CHECK_HIP(hipFree(dv));
        CHECK_HIP(hipFree(dseq));
        CHECK_HIP(hipFree(dpos));
        free(seq);
        free(pos);
    }

    /* the step: append row n-1 and attend over rows [0, n) */
    float *dknew = to_device(k + (size_t)np * row_floats, row_floats * sizeof(float));
    float *dvnew = to_device(v + (size_t)np * row_floats, row_floats * sizeof(float));
    float *dq = to_device(q, (size_t)hq * d * sizeof(float));
    int64_t *dlen = to_device(&n, sizeof(int64_t));
    float *dout = NULL;
    CHECK_HIP(hipMalloc((void **)&dout, (size_t)hq * d * sizeof(float)));
    const size_t ws_bytes = kvq_decode_workspace_bytes(&L, hq, 1, n);
    void *ws = NULL;
    if (ws_bytes == 0) {
        fprintf(stderr, "kvq_decode_workspace_bytes: invalid sizes\n");
        return 3;
    }
    CHECK_HIP(hipMalloc(&ws, ws_bytes));
    CHECK_KVQ(kvq_append_attend_decode(&L, dknew, dvnew, dq, dlen, 1, hq, n, scale, dout, ws, ws_bytes,
                                       status + 1, s));
    CHECK_HIP(hipStreamSynchronize(s));

    float *out = malloc((size_t)hq * d * sizeof(float));
    int32_t st[2];
    CHECK_HIP(hipMemcpy(out, dout, (size_t)hq * d * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(st, status, sizeof st, hipMemcpyDeviceToHost));
    char path[4096];
    snprintf(path, sizeof path, "%s/out.f32", dir);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(out, sizeof(float), (size_t)hq * d, f) != (size_t)hq * d) {
        fprintf(stderr, "%s: write failed\n", path);
        return 4;
    }
    fclose(f);
    printf("append status %d, decode status %d, workspace %zu bytes\n", st[0], st[1], ws_bytes);
    return st[0] != 0 || st[1] != 0 ? 5 : 0;
}
