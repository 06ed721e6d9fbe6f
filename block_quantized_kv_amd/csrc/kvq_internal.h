// kvq_internal.h -- launcher interface between the C ABI (kvq_api.cpp) and the
// HIP kernels.  All arguments are validated by the caller before a launcher
// runs; launchers only enqueue work and return the HIP status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_layout.h"

namespace kvq {

// Stored in a call's dev_status by the attention kernels when a dequantized
// K or V value they read exceeds the binary16 range (KVQ_EOVERFLOW).
constexpr int32_t kStatusOverflow = 6;
// Stored by the fused append + decode when a wave's bounded wait for the
// appending wave's stores ran out (KVQ_EWAIT).
constexpr int32_t kStatusWaitExpired = 7;

// Device view of one plane for one sequence-major layout.
struct PlaneView {
    uint8_t *codes;
    uint16_t *scales;
    int codec;
    int head_dim;
    int n_kv_heads;
    int n_seqs;
    int64_t capacity;
    int64_t head_code_stride;   // bytes per (seq, head)   = capacity/32 * block_code_bytes
    int64_t head_scale_stride;  // binary16 per (seq, head) = capacity/32 * block_scales
};

// Paged planes: the planes are a pool of pages (PlaneView.n_seqs = pages,
// capacity = rows per page); row r of sequence b lives in page
// table[b * table_stride + r / page_rows] at row r % page_rows.
// table == nullptr: contiguous planes (sequence b is "page" b).
struct PageTable {
    const int32_t *table;
    int table_stride;        // entries per sequence
    int page_rows;           // multiple of 32
    int n_seqs;              // sequences (rows of the table)
};

// Both planes of a layer are appended by one launch (grid.y = plane).
struct AppendArgs {
    PlaneView plane[2];      // K, V
    PageTable pt;
    const float *x[2];       // [n_tokens][n_kv_heads][head_dim]; null = skip that plane
    const int32_t *seq_idx;  // [n_tokens]
    const int64_t *pos;      // [n_tokens]
    int n_tokens;
    int32_t *dev_status;     // nullable
};

struct DequantArgs {
    PlaneView plane;
    int role;
    int seq;
    int64_t row0;
    int64_t n_rows;
    float *out;  // [n_kv_heads][n_rows][head_dim]
};

struct DecodeArgs {
    PlaneView k, v;
    PageTable pt;
    // q and out hold q_len consecutive queries per sequence ([q_len][Hq][D] at
    // q + b * q_seq_stride); query i of sequence b sits at row
    // len_b - 1 - q_tail - (q_len - 1 - i) and attends rows up to it.
    const float *q;
    const int64_t *seq_len;  // [n_seqs]
    float *out;
    float *part_o;           // [n_seqs][q_len][Hq][max_splits][D]
    float *part_ml;          // [n_seqs][q_len][Hq][max_splits][2]  (max in log2 units, sum)
    int n_seqs;
    int n_q_heads;
    int gqa;                 // q-heads per kv-head
    int q_len;               // queries per sequence in this launch (gqa * q_len <= 16)
    int q_tail;              // later queries of the same sequences (other launches)
    int64_t q_seq_stride;    // floats between sequences in q and out
    int64_t max_len;
    int split_rows;          // multiple of 256
    int max_splits;
    float scale_log2;        // softmax_scale * log2(e)
    // fused append (app_rows = 0: none): rows len_b - app_rows .. len_b - 1
    // (those at positions >= 0) of every kv-head are first quantized into the
    // cache from app_k / app_v, fp32 [n_seqs][app_rows][n_kv_heads][D]
    const float *app_k;
    const float *app_v;
    int app_rows;
    int32_t *dev_status;     // nullable: kStatusOverflow / kStatusWaitExpired
    // bounded wait of the fused append (polls of the appending wave's flag),
    // and, for tests of its expiry only, a switch that keeps the flag down
    int append_wait_polls;
    int hold_append_flag;
};

// The fused append's wait bound and its test switch (kvq_debug_append_wait).
void set_append_wait(int polls, int hold_flag);
void get_append_wait(int *polls, int *hold_flag);

struct PrefillArgs {
    PlaneView k, v;
    PageTable pt;            // table null: contiguous planes
    const uint16_t *q;       // [T][Hq][D] bf16 bits
    float *out;              // [T][Hq][D]
    int seq;
    int64_t pos0;
    int n_tokens;
    int n_q_heads;
    int gqa;
    float scale_log2;
    int32_t *dev_status;     // nullable: kStatusOverflow when a K_hat / V_hat beyond binary16 is met
};

// Decode split size (rows per workgroup) and split count for a call.
struct DecodePlan {
    int split_rows;
    int max_splits;
    size_t part_o_bytes;
    size_t part_ml_bytes;
    // byte offsets inside the workspace
    size_t off_part_ml, off_part_o, total_bytes;
};
DecodePlan plan_decode(int head_dim, int n_kv_heads, int n_q_heads, int n_seqs, int64_t max_len,
                       int q_len);

// The device scratch of the no-allocation decode entry point: a file-scope
// array of kStaticScratchBytes in the library's code object, one copy per
// GPU.  static_scratch() returns its address on the GPU that `s` runs on
// (looked up once per GPU with that GPU current, then cached).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(hipStream_t s, void **ptr);

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
bool append_supported(int k_codec, int v_codec);
hipError_t launch_dequant(const DequantArgs &a, hipStream_t s);
// Returns hipErrorInvalidValue when no kernel instance exists for the codec
// pair / head_dim (the API maps that to KVQ_EUNSUPPORTED before calling).
bool decode_supported(int k_codec, int v_codec, int head_dim);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
bool prefill_supported(int k_codec, int v_codec, int head_dim);
// Pages of one sequence a paged prefill can address (its workgroups keep the
// sequence's page numbers in LDS).
constexpr int kPrefillMaxPages = 4096;
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

}  // namespace kvq
