/* kvq_probe.h -- on-box measurement helper of libkvq.so (not part of the
 * attention path).  The decode kernel's HBM roofline is reported against the
 * published 8 TB/s peak and against what a plain streaming read reaches on the
 * same GPU; this call is that streaming read. */
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

#ifdef __cplusplus
}
#endif
