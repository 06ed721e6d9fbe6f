/* kvq_probe.h -- measurement helpers (the GPU's own rates), built as their own library
 * (libkvq_probe.so), not part of the attention path and not linked into
 * libkvq.so.  The decode kernel's HBM roofline is reported against the
 * published 8 TB/s peak and against what a plain streaming read reaches on the
 * same GPU; the prefill kernel's matrix-core roofline against the published
 * dense peak and against what a plain loop of its own product instruction
 * reaches.  These two calls are those measurements. */
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of device memory at `buf` once, with n_workgroups workgroups
 * of 8 waves; each wave reads one contiguous stripe of bytes / (8 *
 * n_workgroups) bytes, which must be a positive multiple of 8 KiB (and bytes
 * < 2 GiB).  `sink` (one device uint32) is written only on an impossible
 * match, so the kernel has no visible effect.  Enqueues one kernel on
 * hip_stream and returns without waiting; KVQ_EINVAL for sizes that do not
 * divide as stated, KVQ_EHIP if the launch fails. */
kvq_status kvq_probe_stream_read(const void *buf, size_t bytes, int32_t n_workgroups, uint32_t *sink,
                                 void *hip_stream);

/* Runs n_workgroups workgroups of 8 waves; each wave issues iters x 8
 * independent v_mfma_f32_16x16x32_f16 products (16384 flop each) from
 * registers.  *flop (host, nullable) receives the flop count of the launch.
 * `sink` as above.  Enqueues one kernel and returns without waiting; KVQ_EINVAL
 * for a null sink or non-positive sizes, KVQ_EHIP if the launch fails. */
kvq_status kvq_probe_mfma_f16(int32_t n_workgroups, int32_t iters, uint32_t *sink, double *flop,
                              void *hip_stream);

#ifdef __cplusplus
}
#endif
