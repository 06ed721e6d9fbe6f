"""block_quantized_kv_amd -- attention over a block-quantized KV cache on MI355X.

The compute path is the HIP library ``libkvq.so`` (C ABI in include/kvq.h);
this package is a thin ctypes binding over it with the same entry-point names
(argument marshalling only).  PyTorch provides device memory and streams.

There is no CPU or PyTorch fallback: importing the binding without the built
library raises.
"""
from ._binding import (  # noqa: F401
    BLOCK_ROWS,
    CODECS,
    KVQ_EOVERFLOW,
    KVQ_EWAIT,
    KvqError,
    Plane,
    Layer,
    PagedLayer,
    kvq_append,
    kvq_append_attend_decode,
    kvq_append_attend_decode_mq,
    kvq_append_attend_decode_noalloc,
    kvq_noalloc_scratch_bytes,
    kvq_attend_decode,
    kvq_attend_decode_mq,
    kvq_attend_prefill,
    kvq_dequant,
    kvq_debug_append_wait,
    kvq_decode_workspace_bytes,
    decode_workspace,
    decode_mq_workspace,
    kvq_decode_mq_workspace_bytes,
    kvq_prefill_workspace_bytes,
    kvq_paged_append,
    kvq_paged_attend_decode_mq,
    kvq_paged_append_attend_decode_mq,
    kvq_paged_attend_prefill,
    kvq_paged_decode_workspace_bytes,
    paged_decode_workspace,
    kvq_plane_bytes,
    kvq_row_code_bytes,
    kvq_status_str,
    kvq_last_error,
    library_path,
    load_library,
)
