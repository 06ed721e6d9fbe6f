// stream_probe.hip -- measured streaming-read rate, the practical ceiling that
// the decode kernel's HBM roofline is quoted against beside the published
// peak.  Not part of the attention path.
//
// Each wave reads a contiguous stripe of the buffer with 16-byte
// non-temporal buffer loads (the decode kernel's cache policy), eight 1 KB
// pieces in flight, and folds the words into one value that
// is stored only if it matches an impossible pattern (so the loads stay).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
constexpr int kWavesPerGroup = 8;
constexpr int kDepth = 8;              // 1 KB pieces in flight per wave
constexpr uint32_t kPiece = 1024;

__global__ __launch_bounds__(64 * kWavesPerGroup) void stream_read_kernel(const unsigned char *base, uint32_t bytes,
                                                                         uint32_t per_wave, uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(base), 0, (int)bytes, 0x00020000);
    const uint32_t w0 = wave * per_wave;
    uint32_t acc = 0;
    for (uint32_t off = 0; off < per_wave; off += kDepth * kPiece) {
        u4v v[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d)
            v[d] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, w0 + off + d * kPiece + lane * 16, 0, 2 /* nt */));
#pragma unroll
        for (int d = 0; d < kDepth; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" kvq_status kvq_probe_stream_read(const void *buf, size_t bytes, int32_t n_workgroups, uint32_t *sink,
                                            void *hip_stream) {
    if (!buf || !sink || n_workgroups <= 0) return KVQ_EINVAL;
    const size_t per_wave = bytes / ((size_t)n_workgroups * kWavesPerGroup);
    if (bytes > 0x7fffffffu || per_wave == 0 || per_wave % (kDepth * kPiece) != 0 ||
        per_wave * (size_t)n_workgroups * kWavesPerGroup != bytes)
        return KVQ_EINVAL;
    stream_read_kernel<<<dim3((unsigned)n_workgroups), dim3(64 * kWavesPerGroup), 0,
                         static_cast<hipStream_t>(hip_stream)>>>(static_cast<const unsigned char *>(buf),
                                                                 (uint32_t)bytes, (uint32_t)per_wave, sink);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}
