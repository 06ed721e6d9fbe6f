// attn_prefill.hip -- chunked-prefill attention (placeholder until the bf16
// matrix-core kernel lands: reports "unsupported", never falls back).
#include "kvq_internal.h"

namespace kvq {

bool prefill_supported(int, int, int) { return false; }

hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvq
