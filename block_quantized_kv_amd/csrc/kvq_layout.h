// kvq_layout.h -- codec constants and the in-block permutation of the cache
// planes.  Host and device.
//
// A plane stores, per (sequence, kv-head), blocks of 32 consecutive rows.
// Inside a block, codes and scales sit in the order in which the matrix-core
// kernels read them, so that every wave-wide load is one contiguous run of
// memory and every lane receives exactly its operand bytes:
//
//  K role (operand of S^T = K Q^T, rows on the 16-wide M side): the block is
//   two 16-row tiles.  In a tile, lane L = i + 16*kq (i = row in tile, kq in
//   0..3) owns, for every 32-channel k-step t, the codes of channels
//   32t + 8kq + s, s = 0..7 ("slots").  4-bit codecs: one 32-bit word per
//   k-step, slot s in nibble position slot_nibble(s); q8_0: 8 bytes per
//   k-step in slot order.  A lane's bytes are cut in chunks of W = min(16,
//   lane bytes) and laid out chunk-major: [chunk][lane][W].
//   Scales of a tile: [q][group][r] for row i = 4q + r (q, r in 0..3), which
//   is the row set lane (head, q) holds in the 16x16 accumulator.
//
//  V role (operand of O^T = V^T P^T, channels on the M side, rows as the
//   contraction): lane L = c16 + 16*kq owns, for every 16-channel block cb,
//   the codes of channel 16cb + c16 for the eight rows
//   (s/4)*16 + 4kq + (s%4), s = 0..7 -- exactly the rows whose probabilities
//   the same lane holds after the S^T product.  Same nibble/byte slot order
//   and the same chunk-major layout as K.
//   Scales: [kq][group][s] for those eight rows.
//
//  F16 (no scales): the same lane order with one binary16 value (2 bytes) per
//   slot: 16 bytes per k-step (K) or per channel block (V) and lane, so a
//   lane's 16-byte run is exactly its 8-value matrix-core operand.
//
// The 4-bit slot order (0,4,1,5,2,6,3,7 in nibble positions) is the one in
// which a word splits into binary16 pairs with two masks and one shift.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define KVQ_HD __host__ __device__ __forceinline__
#else
#define KVQ_HD inline
#endif

namespace kvq {

// F16: the f16 control codec (each value its binary16 rounding, 2 bytes, no
// scales), the cache the quantized codecs are measured against.
enum : int { Q8_0 = 0, Q4_0 = 1, Q4_G64 = 2, F16 = 3 };
enum : int { ROLE_K = 0, ROLE_V = 1 };
constexpr int kBlockRows = 32;

// group_size: values per binary16 scale (F16 has no scales; its "group" is
// taken as 32 values so that divisions stay defined, with 0 scales per row)
KVQ_HD constexpr int group_size(int codec) { return codec == Q4_G64 ? 64 : 32; }
KVQ_HD constexpr int qmax(int codec) { return codec == Q8_0 ? 127 : 7; }
KVQ_HD constexpr bool is8(int codec) { return codec == Q8_0; }
KVQ_HD constexpr bool is16(int codec) { return codec == F16; }
KVQ_HD constexpr int row_bytes(int codec, int d) { return is16(codec) ? 2 * d : is8(codec) ? d : d / 2; }
KVQ_HD constexpr int n_groups(int codec, int d) { return is16(codec) ? 0 : d / group_size(codec); }
KVQ_HD constexpr int block_code_bytes(int codec, int d) { return kBlockRows * row_bytes(codec, d); }
KVQ_HD constexpr int block_scales(int codec, int d) { return kBlockRows * n_groups(codec, d); }

// Bytes one lane owns per K tile / per V block.
KVQ_HD constexpr int k_lane_bytes(int codec, int d) { return is16(codec) ? d / 2 : is8(codec) ? d / 4 : d / 8; }
KVQ_HD constexpr int v_lane_bytes(int codec, int d) { return is16(codec) ? d : is8(codec) ? d / 2 : d / 4; }
KVQ_HD constexpr int chunk_width(int lane_bytes) { return lane_bytes < 16 ? lane_bytes : 16; }

// Nibble position (0..7 within a 32-bit word) of MFMA slot s.
KVQ_HD constexpr int slot_nibble(int s) { return (s >> 1) + 4 * (s & 1); }

// Offset of lane byte b of `lane` in a region where each lane owns LB bytes.
KVQ_HD constexpr int lane_byte_offset(int LB, int lane, int b) {
    return (b / chunk_width(LB)) * (64 * chunk_width(LB)) + lane * chunk_width(LB) +
           (b % chunk_width(LB));
}

struct CodePos {
    int byte;   // byte offset inside the block
    int shift;  // 0: low nibble or whole byte, 4: high nibble
};

// Position of the code of row j (0..31) and channel c inside a K-role block.
KVQ_HD CodePos k_code_pos(int codec, int d, int j, int c) {
    const int tau = j >> 4, i = j & 15;
    const int t = c >> 5, kq = (c & 31) >> 3, s = c & 7;
    const int lane = i + 16 * kq;
    const int tile = tau * 16 * row_bytes(codec, d);
    if (is16(codec)) return {tile + lane_byte_offset(k_lane_bytes(codec, d), lane, 16 * t + 2 * s), 0};
    if (is8(codec)) return {tile + lane_byte_offset(k_lane_bytes(codec, d), lane, 8 * t + s), 0};
    const int p = slot_nibble(s);
    return {tile + lane_byte_offset(k_lane_bytes(codec, d), lane, 4 * t + (p >> 1)), 4 * (p & 1)};
}

// Index (in binary16 units) of the scale of row j, group g in a K-role block.
KVQ_HD int k_scale_index(int codec, int d, int j, int g) {
    const int ng = n_groups(codec, d);
    const int tau = j >> 4, i = j & 15;
    return tau * 16 * ng + (i >> 2) * 4 * ng + g * 4 + (i & 3);
}

// V-role lane group and slot of row j.
KVQ_HD constexpr int v_kq(int j) { return (j & 15) >> 2; }
KVQ_HD constexpr int v_slot(int j) { return 4 * (j >> 4) + (j & 3); }

KVQ_HD CodePos v_code_pos(int codec, int d, int j, int c) {
    const int cb = c >> 4, c16 = c & 15;
    const int lane = c16 + 16 * v_kq(j), s = v_slot(j);
    if (is16(codec)) return {lane_byte_offset(v_lane_bytes(codec, d), lane, 16 * cb + 2 * s), 0};
    if (is8(codec)) return {lane_byte_offset(v_lane_bytes(codec, d), lane, 8 * cb + s), 0};
    const int p = slot_nibble(s);
    return {lane_byte_offset(v_lane_bytes(codec, d), lane, 4 * cb + (p >> 1)), 4 * (p & 1)};
}

KVQ_HD int v_scale_index(int codec, int d, int j, int g) {
    const int ng = n_groups(codec, d);
    return v_kq(j) * 8 * ng + g * 8 + v_slot(j);
}

}  // namespace kvq
