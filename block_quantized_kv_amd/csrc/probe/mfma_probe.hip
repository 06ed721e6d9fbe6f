// mfma_probe.hip -- measured matrix-core throughput of v_mfma_f32_16x16x32_f16,
// the instruction the prefill kernel's products run on: the practical ceiling
// its MFMA roofline is quoted against beside the published dense peak.  Not
// part of the attention path.
//
// Every wave keeps kChains independent accumulator chains (enough to cover
// the instruction's latency) and issues `iters` rounds of one product per
// chain from operands held in registers; the accumulators are folded into
// one value that is stored only if it matches an impossible pattern, so the
// products stay.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kWaves = 8;
constexpr int kChains = 8;

__global__ __launch_bounds__(64 * kWaves) void mfma_f16_kernel(int iters, float seed, uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    h8v a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(seed * (float)(lane + i));
        b[i] = (_Float16)(seed * (float)(lane - i));
    }
    f4v acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4v{0.f, 0.f, 0.f, (float)c};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (__builtin_bit_cast(uint32_t, s) == 0x7fbadbadu) sink[0] = 1u;
}

}  // namespace

extern "C" kvq_status kvq_probe_mfma_f16(int32_t n_workgroups, int32_t iters, uint32_t *sink, double *flop,
                                         void *hip_stream) {
    if (!sink || n_workgroups <= 0 || iters <= 0) return KVQ_EINVAL;
    mfma_f16_kernel<<<dim3((unsigned)n_workgroups), dim3(64 * kWaves), 0, static_cast<hipStream_t>(hip_stream)>>>(
        iters, 1.0f / 1024.0f, sink);
    if (flop) *flop = (double)n_workgroups * kWaves * (double)iters * kChains * (2.0 * 16 * 16 * 32);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}
